// Device-side helpers shared by the libtsp kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace tsp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Shape bundle passed by value to kernels (derived quantities precomputed on
// the host so kernels do no divisions they can avoid).
struct Shape {
  int32_t B, S, D, r, h, Hq, Hkv, dh, F;
  int32_t part;  // token partition: 0 zigzag, 1 striped
  int32_t T, c, M, Hq_s, Hkv_s, F_s, kmax, kmax_pad, nqkv_s;
};

// Compile-time loop: f(integral_constant<int, J>) for J = J0 .. N-1.
template <int J, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (J < N) {
    f(std::integral_constant<int, J>{});
    static_for<J + 1, N>(f);
  }
}
template <int V>
using IC = std::integral_constant<int, V>;

// 32x32x16 matrix-core products (float32 accumulate).  Operand i-index is
// the lane's low 5 bits, the 8 k-values live in the lane's 16 bytes; the
// result lane l, register v holds row 8*(v/4) + 4*(l/32) + v%4, column l%32.
__device__ __forceinline__ f32x16 mfma_bf16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(const u32x4& a, const u32x4& b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two packed bfloat16 -> two packed f16, round to nearest even (exact for
// every bfloat16 inside the f16 normal range; tiny values lose low bits).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  float lo = __uint_as_float(u << 16);
  float hi = __uint_as_float(u & 0xffff0000u);
  f16x2 r;
  r[0] = (_Float16)lo;
  r[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 v) {
  u32x4 o;
  o[0] = bf16x2_to_f16x2(v[0]);
  o[1] = bf16x2_to_f16x2(v[1]);
  o[2] = bf16x2_to_f16x2(v[2]);
  o[3] = bf16x2_to_f16x2(v[3]);
  return o;
}

__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f16x2 r;
  r[0] = (_Float16)a;
  r[1] = (_Float16)b;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(((uint32_t)u) << 16);
}

}  // namespace tsp
