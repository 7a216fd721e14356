// Host-only stand-ins for libtsp's kernel launchers, so that the C ABI's
// argument checks, workspace sizing and dispatch logic (tsp_abi.cpp) can be
// built and run under AddressSanitizer / UndefinedBehaviorSanitizer on a
// machine without a GPU.  Test infrastructure only: nothing here runs on a
// device.  The attention work plan has its own sanitized check
// (attn_plan_check.cpp); here its workspace size is a fixed stand-in.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace tsp {
hipError_t launch_zigzag_index(const Shape&, int32_t*, int32_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_kv_reorder(const Shape&, const uint16_t*, uint16_t*, uint16_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_qkv_gemm(const Shape&, int, const uint16_t*, const uint16_t*, uint16_t*, uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_oproj_gemm(const Shape&, const uint16_t*, const uint16_t*, const uint16_t*, const float*, float*,
                             uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_gateup_gemm(const Shape&, const uint16_t*, bool, const uint16_t*, const uint16_t*, uint16_t*,
                              hipStream_t, float*) {
  return hipSuccess;
}
hipError_t launch_down_gemm(const Shape&, const uint16_t*, const uint16_t*, const float*, float*, float*,
                            hipStream_t) {
  return hipSuccess;
}
hipError_t launch_f32_to_f16(const float*, uint16_t*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_transpose_bf16(int, const void*, int64_t, int64_t, uint16_t*, int64_t, int64_t, int, int, int, int,
                                 hipStream_t) {
  return hipSuccess;
}
hipError_t launch_f32_to_bf16(const float*, uint16_t*, int64_t, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_da(const Shape&, const uint16_t*, const uint16_t*, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_da_kept(const Shape&, const uint16_t*, const uint16_t*, const float*, uint16_t*, uint16_t*,
                              hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_gu(const Shape&, const uint16_t*, bool, const uint16_t*, const uint16_t*, const float*,
                         uint16_t*, uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_dx(const Shape&, const uint16_t*, const uint16_t*, const float*, float*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_dwd(const Shape&, int, const uint16_t*, const uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_dwgu(const Shape&, int, const uint16_t*, const uint16_t*, float*, float*, hipStream_t) {
  return hipSuccess;
}
bool kmajor_ok(const Shape& s, int use) { return use != KMAJ_DX_MLP || s.F_s % 32 == 0; }
hipError_t launch_bwd_da_kmajor(const Shape&, const uint16_t*, const uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_da_kept_kmajor(const Shape&, const uint16_t*, const uint16_t*, const float*, uint16_t*,
                                     uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_dx_kmajor(const Shape&, const uint16_t*, const uint16_t*, const uint16_t*, const float*, float*,
                                float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_do_kmajor(const Shape&, const uint16_t*, const uint16_t*, uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_dx_kmajor(const Shape&, const uint16_t*, const uint16_t*, const float*, float*, float*,
                                     hipStream_t) {
  return hipSuccess;
}
AttnPlan attn_plan(const Shape&) { return AttnPlan{}; }
size_t attn_partial_bytes(const Shape& s) { return (size_t)s.M * s.Hq * (s.dh + 2) * 4; }
AttnPlan attn_plan_shape(const Shape&, int) { return AttnPlan{}; }
hipError_t launch_flash_attn(const Shape&, const uint16_t*, const uint16_t*, uint16_t*, float*, hipStream_t, float*) {
  return hipSuccess;
}
hipError_t launch_copy_bf16(int, const void*, int64_t, int64_t, uint16_t*, int64_t, int64_t, int, int, int,
                            hipStream_t) {
  return hipSuccess;
}
hipError_t launch_q_gemm(const Shape&, const uint16_t*, const uint16_t*, uint16_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_attn_bwd_do(const Shape&, const uint16_t*, const uint16_t*, uint16_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_dwo(const Shape&, int, const uint16_t*, const uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_dx(const Shape&, const uint16_t*, const uint16_t*, const float*, float*, float*,
                              hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_dwqkv(const Shape&, int, const uint16_t*, const uint16_t*, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_attn_bwd_core(const Shape&, const uint16_t*, const uint16_t*, const uint16_t*, const uint16_t*,
                                const float*, float*, float*, float*, float*, hipStream_t) {
  return hipSuccess;
}
}  // namespace tsp
