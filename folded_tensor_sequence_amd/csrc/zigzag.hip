// Token partition maps and the K/V reorder into sequence order (gfx950).
//
// Zigzag partition (Zyphra TSP article on ai-trends.today, section "How to
// Fold a Book": the gathered K/V are put back in sequence order with a zigzag
// partition chosen to balance causal attention work across ranks;
// r007.github.io "Распределенное обучение", section "Параллелизм по
// контексту: Ring Attention против Ulysses", item 1): the S positions form 2D
// chunks of c = S/(2D); rank r holds chunk r, then chunk 2D-1-r.  Striped
// partition (the alternative that item names): position g lives on rank
// g mod D at local row g div D.
#include "common.h"
#include "kernels.h"

namespace tsp {

__device__ __forceinline__ int32_t zz_local_to_global(int32_t t, int32_t c, int32_t D, int32_t r) {
  return t < c ? r * c + t : (2 * D - 1 - r) * c + (t - c);
}

// Slot rank*T + t of global position g in a rank-major all-gather.
__device__ __forceinline__ int32_t zz_global_to_slot(int32_t g, int32_t c, int32_t D, int32_t T) {
  int32_t q = g / c, i = g - q * c;
  return q < D ? q * T + i : (2 * D - 1 - q) * T + c + i;
}

// Rank and local row of global position g under the shape's partition.
__device__ __forceinline__ void part_owner(const Shape& s, int32_t g, int32_t& src, int32_t& t) {
  if (s.part == 1) {
    src = g % s.D;
    t = g / s.D;
  } else {
    const int32_t q = g / s.c, i = g - q * s.c;
    src = q < s.D ? q : 2 * s.D - 1 - q;
    t = q < s.D ? i : s.c + i;
  }
}

__global__ void zigzag_index_kernel(Shape s, int32_t* __restrict__ l2g, int32_t* __restrict__ g2s) {
  int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < s.T) l2g[i] = s.part == 1 ? i * s.D + s.r : zz_local_to_global(i, s.c, s.D, s.r);
  if (g2s != nullptr && i < s.S) {
    if (s.part == 1) {
      int32_t src, t;
      part_owner(s, i, src, t);
      g2s[i] = src * s.T + t;
    } else {
      g2s[i] = zz_global_to_slot(i, s.c, s.D, s.T);
    }
  }
}

hipError_t launch_zigzag_index(const Shape& s, int32_t* l2g, int32_t* g2s, hipStream_t st) {
  int n = s.S > s.T ? s.S : s.T;
  dim3 grid((n + 255) / 256);
  hipLaunchKernelGGL(zigzag_index_kernel, grid, dim3(256), 0, st, s, l2g, g2s);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// K/V reorder.  One block moves a tile of 64 natural-order keys of one
// (kv-head, sequence, K-or-V) triple.  Thread (kc, dc) owns keys 8*kc..+7 and
// head-dim columns 8*dc..+7: it reads eight 16-byte row pieces (one per key)
// and writes them unchanged (K, key-major) or transposed in registers (V,
// dh-major), so both the reads and the writes of a wave cover whole 128-byte
// runs.  Keys in [kmax, kmax_pad) are written as zeros.
// --------------------------------------------------------------------------
template <int DH>
__global__ __launch_bounds__(8 * (DH / 8)) void kv_reorder_kernel(
    Shape s, const uint16_t* __restrict__ gathered, uint16_t* __restrict__ knat,
    uint16_t* __restrict__ vnat) {
  constexpr int NDC = DH / 8;
  const int tid = threadIdx.x;
  const int kc = tid % 8;  // key chunk (fastest: writes of V rows are contiguous)
  const int dc = tid / 8;  // head-dim chunk
  const int ntiles = s.kmax_pad / 64;
  int bid = blockIdx.x;
  const int tile = bid % ntiles;
  bid /= ntiles;
  const int kv = bid % 2;
  bid /= 2;
  const int b = bid % s.B;
  const int G = bid / s.B;           // global kv head
  const int j = G / s.Hkv_s;         // shard
  const int hk = G - j * s.Hkv_s;    // head within shard
  const int64_t row_elems = (int64_t)s.Hkv_s * DH;

  // Source rows of the thread's 8 keys.  Zigzag with c % 8 == 0: the 8 keys
  // sit in one chunk at consecutive local rows (one address, fixed stride),
  // and all of them are copied when the group lies below kmax (a kmax that
  // is not a multiple of 8 ends inside a group: that group takes the per-key
  // path, which zero-fills the keys past kmax); otherwise each key's rank
  // and row are computed on their own.
  const int g0 = tile * 64 + kc * 8;
  const uint16_t* col = gathered + (int64_t)hk * DH + dc * 8;
  const int64_t src_base = (((int64_t)j * s.D * 2 + kv) * s.B + b) * s.T;  // row of (src 0, t 0)
  const int64_t src_step = (int64_t)2 * s.B * s.T;                          // rows per src rank
  u32x4 v[8];
  if (s.part == 0 && s.c % 8 == 0 && (g0 + 8 <= s.kmax || g0 >= s.kmax)) {
    if (g0 < s.kmax) {
      const int q = g0 / s.c, i = g0 - q * s.c;
      const int src = q < s.D ? q : 2 * s.D - 1 - q;
      const int t = q < s.D ? i : s.c + i;
      const uint16_t* p = col + (src_base + src * src_step + t) * row_elems;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = *reinterpret_cast<const u32x4*>(p + e * row_elems);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = u32x4{0u, 0u, 0u, 0u};
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (g0 + e < s.kmax) {
        int src, t;
        part_owner(s, g0 + e, src, t);
        v[e] = *reinterpret_cast<const u32x4*>(col + (src_base + src * src_step + t) * row_elems);
      } else {
        v[e] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  const int64_t head = (int64_t)G * s.B + b;
  if (kv == 0) {
    uint16_t* base = knat + head * s.kmax_pad * DH;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int g = tile * 64 + kc * 8 + e;
      *reinterpret_cast<u32x4*>(base + (int64_t)g * DH + dc * 8) = v[e];
    }
  } else {
    // 8x8 transpose of 16-bit values: out[d][k] = in[k][d].
    uint16_t* base = vnat + head * (int64_t)DH * s.kmax_pad;
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      const int w = d / 2;
      const bool hi = d & 1;
      u32x4 o;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        uint32_t a = v[2 * p][w], c2 = v[2 * p + 1][w];
        uint32_t lo16 = hi ? (a >> 16) : (a & 0xffffu);
        uint32_t hi16 = hi ? (c2 & 0xffff0000u) : (c2 << 16);
        o[p] = lo16 | hi16;
      }
      *reinterpret_cast<u32x4*>(base + (int64_t)(dc * 8 + d) * s.kmax_pad + tile * 64 + kc * 8) = o;
    }
  }
}

hipError_t launch_kv_reorder(const Shape& s, const uint16_t* gathered, uint16_t* knat,
                             uint16_t* vnat, hipStream_t st) {
  const int ntiles = s.kmax_pad / 64;
  dim3 grid((unsigned)ntiles * 2u * (unsigned)s.B * (unsigned)s.Hkv);
  if (s.dh == 128) {
    hipLaunchKernelGGL(kv_reorder_kernel<128>, grid, dim3(128), 0, st, s, gathered, knat, vnat);
  } else {
    hipLaunchKernelGGL(kv_reorder_kernel<64>, grid, dim3(64), 0, st, s, gathered, knat, vnat);
  }
  return hipGetLastError();
}

}  // namespace tsp
