// Internal launchers of libtsp (host side).  Each returns the HIP error of
// its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace tsp {

hipError_t launch_zigzag_index(const Shape& s, int32_t* l2g, int32_t* g2s, hipStream_t st);
hipError_t launch_kv_reorder(const Shape& s, const uint16_t* gathered, uint16_t* knat,
                             uint16_t* vnat, hipStream_t st);

// Packed Q/K/V projection of src_rank's tokens (bf16 matrix cores).
hipError_t launch_qkv_gemm(const Shape& s, int src_rank, const uint16_t* x, const uint16_t* w_qkv,
                           uint16_t* q, uint16_t* kv_gathered, hipStream_t st);

// out = x(bf16) + O * W_o^T over the D shards' K-segments; also an f16 copy
// of out when out16 != nullptr.
hipError_t launch_oproj_gemm(const Shape& s, const uint16_t* o, const uint16_t* w_o,
                             const uint16_t* x_resid, float* out, uint16_t* out16, hipStream_t st);

// act = silu(h16 Wg^T) * (h16 Wu^T) (f16 matrix cores, weights bf16->f16).
hipError_t launch_gateup_gemm(const Shape& s, const uint16_t* h16, const uint16_t* w_g,
                              const uint16_t* w_u, uint16_t* act, hipStream_t st);

// y = resid + sum over ring steps of act_j W_d,j^T.
hipError_t launch_down_gemm(const Shape& s, const uint16_t* act, const uint16_t* w_d,
                            const float* resid, float* y, hipStream_t st);

// f32 -> f16 rounding copy (MLP input when it arrives as float32).
hipError_t launch_f32_to_f16(const float* x, uint16_t* y, int64_t n, hipStream_t st);

// Causal flash attention over the natural-order K/V.
hipError_t launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* knat,
                             const uint16_t* vnat, uint16_t* o, hipStream_t st);

}  // namespace tsp
