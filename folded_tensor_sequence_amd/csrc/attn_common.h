// Device helpers shared by the attention kernels (forward and backward).
#pragma once

#include "common.h"

namespace tsp {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// 16-byte (and, with bytes = 4, 4-byte) copy global -> LDS: lane i's bytes
// land at the instruction's LDS base + i * bytes.
__device__ __forceinline__ void attn_load_lds16(const uint16_t* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void attn_load_lds4(const float* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, 0);
}

// Row of the all-gathered K/V buffer holding global position p.  Zigzag:
// chunk q = p / c lives on rank q (q < D) or 2D-1-q, at local row p mod c
// (+ c for the later chunk).  Striped: rank p mod D, local row p div D.
__device__ __forceinline__ int64_t gathered_row(const Shape& s, int j, int sel, int b, int p) {
  int g, t;
  if (s.part == 1) {
    g = p % s.D;
    t = p / s.D;
  } else {
    const int qc = p / s.c;
    g = qc < s.D ? qc : 2 * s.D - 1 - qc;
    t = (qc < s.D ? 0 : s.c) + (p - qc * s.c);
  }
  return ((((int64_t)j * s.D + g) * 2 + sel) * s.B + b) * s.T + t;
}

// Global position of the rank's local row t (zigzag: chunks r and 2D-1-r;
// striped: t D + r).  Increasing in t for both partitions.
__device__ __forceinline__ int local_pos(const Shape& s, int t) {
  const int zz = t < s.c ? s.r * s.c + t : (2 * s.D - 1 - s.r) * s.c + (t - s.c);
  return s.part == 1 ? t * s.D + s.r : zz;
}

// The rank's first local row whose position is >= p (T when none is).
__device__ __forceinline__ int first_row_from(const Shape& s, int p) {
  if (s.part == 1) {
    if (p <= s.r) return 0;
    const int t = (p - s.r + s.D - 1) / s.D;
    return t < s.T ? t : s.T;
  }
  const int a0 = s.r * s.c, b0 = (2 * s.D - 1 - s.r) * s.c;
  if (p <= a0) return 0;
  if (p < a0 + s.c) return p - a0;
  if (p <= b0) return s.c;
  if (p < b0 + s.c) return s.c + (p - b0);
  return s.T;
}

}  // namespace tsp
