// Causal flash attention of one rank's zigzag queries over the natural-order
// K/V (gfx950, f16 matrix cores, float32 online softmax).
//
// Zyphra TSP article on ai-trends.today, section "How to Fold a Book": after
// the all-gather and the zigzag reorder, every rank runs attention of its own
// tokens against the whole K/V context.  Blockwise attention keeps a running
// row maximum and row sum and rescales the partial output when the maximum
// grows (r007.github.io "Распределенное обучение", section "Параллелизм по
// контексту: Ring Attention против Ulysses": the online-softmax accumulator),
// so the S x S score matrix is never stored.
//
// Work item = (sequence b, q-head, block of 128 local rows inside one zigzag
// chunk); 4 waves x 32 query rows.  Items of the later chunk (longer key
// prefix) come first in the grid so the dispatcher hands out the long ones
// first.  Per 64-key tile:
//   S^T = K Q^T   (32x32x16 MFMA, K from LDS as the first operand, the wave's
//                  Q rows kept in registers as the second) -> each lane holds
//                  one query (column) and 32 of the tile's 64 keys; the lane
//                  pair (l, l^32) shares a query, so row max/sum need only one
//                  cross-half exchange.
//   K rows are stored in LDS in a permuted order so that, for every 16-key
//   step of the P V product, a lane's 8 probabilities are 8 consecutive keys;
//   V is stored transposed (head-dim major) so those 8 keys are one 16-byte
//   LDS read.
//   O^T += V^T P  (32x32x16 MFMA, probabilities rounded to f16).
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace tsp {

struct AttnArgs {
  const uint16_t* q;     // f16 [B][Hq][T][dh]
  const uint16_t* knat;  // f16 [Hkv][B][kmax_pad][dh]
  const uint16_t* vnat;  // f16 [Hkv][B][dh][kmax_pad]
  uint16_t* o;           // f16 [B][T][Hq*dh]
  Shape s;
  float scale_log2;      // log2(e) / sqrt(dh)
  int32_t nrb;           // 128-row blocks per chunk
};

// Row permutation inside each 32-key group: swaps 4-row blocks 1<->2, 5<->6.
__device__ __forceinline__ int key_perm(int i) {
  const int b4 = (i >> 2) & 7;
  return ((b4 ^ (b4 >> 1)) & 1) ? (i ^ 12) : i;
}

template <int DH>
__global__ __launch_bounds__(256, 2) void flash_attn_kernel(AttnArgs a) {
  constexpr int BN = 64;
  constexpr int KROW = DH * 2;
  constexpr int K_BYTES = BN * KROW;
  constexpr int V_BYTES = DH * BN * 2;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int KCH = DH / 8;
  constexpr int K_LD = BN * KCH / 256;
  constexpr int V_LD = DH * 8 / 256;
  constexpr int NDB = DH / 32;
  constexpr int NKS = DH / 16;
  __shared__ __align__(16) unsigned char smem[2 * STAGE];

  const Shape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lrow = lane & 31, lgrp = lane >> 5;

  // ---- work item -------------------------------------------------------
  const int per = s.B * s.Hq;
  const int pos = blockIdx.x / per, bh = blockIdx.x - pos * per;
  const int b = bh / s.Hq, qh = bh - b * s.Hq;
  const int late = pos < a.nrb ? 1 : 0;
  const int rb = a.nrb - 1 - (late ? pos : pos - a.nrb);
  const int row_begin = late * s.c, row_end = row_begin + s.c;
  const int gstart = (late ? (2 * s.D - 1 - s.r) : s.r) * s.c;
  const int t0 = row_begin + rb * 128;
  const int wt0 = t0 + wave * 32;
  const bool wave_active = wt0 < row_end;
  int t_lane = wt0 + lrow;
  const bool lane_valid = t_lane < row_end;
  t_lane = lane_valid ? t_lane : row_end - 1;
  const int qpos = gstart + (t_lane - row_begin);
  const int wg_last = (t0 + 127 < row_end ? t0 + 127 : row_end - 1);
  const int nkt = (gstart + (wg_last - row_begin) + BN) / BN;
  const int w_last = (wt0 + 31 < row_end ? wt0 + 31 : row_end - 1);
  const int wave_maxpos = gstart + (w_last - row_begin);
  const int wave_minpos = gstart + (wt0 - row_begin);

  const int G = qh / (s.Hq / s.Hkv);
  const uint16_t* kbase = a.knat + ((int64_t)G * s.B + b) * s.kmax_pad * DH;
  const uint16_t* vbase = a.vnat + ((int64_t)G * s.B + b) * DH * (int64_t)s.kmax_pad;

  // ---- Q fragments (second operand of S^T = K Q^T) ---------------------
  u32x4 qf[NKS];
  {
    const uint16_t* qrow = a.q + (((int64_t)b * s.Hq + qh) * s.T + t_lane) * DH;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + lgrp * 8);
  }

  // ---- K/V tile staging -------------------------------------------------
  u32x4 rk[K_LD], rv[V_LD];
  auto gload = [&](int kt) {
    const int key0 = kt * BN;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int ci = tid + 256 * i, kr = ci / KCH, kc = ci - kr * KCH;
      rk[i] = *reinterpret_cast<const u32x4*>(kbase + (int64_t)(key0 + kr) * DH + kc * 8);
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int ci = tid + 256 * i, d = ci >> 3, vc = ci & 7;
      rv[i] = *reinterpret_cast<const u32x4*>(vbase + (int64_t)d * s.kmax_pad + key0 + vc * 8);
    }
  };
  auto lstore = [&](int stage) {
    unsigned char* sk = smem + stage * STAGE;
    unsigned char* sv = sk + K_BYTES;
#pragma unroll
    for (int i = 0; i < K_LD; ++i) {
      const int ci = tid + 256 * i, kr = ci / KCH, kc = ci - kr * KCH;
      const int row = (kr & ~31) | key_perm(kr & 31);
      *reinterpret_cast<u32x4*>(sk + row * KROW + ((kc ^ (row & 7)) << 4)) = rk[i];
    }
#pragma unroll
    for (int i = 0; i < V_LD; ++i) {
      const int ci = tid + 256 * i, d = ci >> 3, vc = ci & 7;
      *reinterpret_cast<u32x4*>(sv + d * 128 + ((vc ^ (d & 7)) << 4)) = rv[i];
    }
  };

  f32x16 oacc[NDB];
#pragma unroll
  for (int x = 0; x < NDB; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[x][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;
  const float sc = a.scale_log2;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + 1 < nkt) gload(kt + 1);
    const int key0 = kt * BN;
    if (wave_active && key0 <= wave_maxpos) {
      const unsigned char* sk = smem + (kt & 1) * STAGE;
      const unsigned char* sv = sk + K_BYTES;
      f32x16 sacc[2];
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[x][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int pch = ((2 * ks + lgrp) ^ (lrow & 7)) << 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + (kb * 32 + lrow) * KROW + pch);
          sacc[kb] = mfma_f16(kf, qf[ks], sacc[kb]);
        }
      }
      // causal mask: register v of key group kb is key key0 + 32kb + 16(v/8) + 8 lgrp + v%8
      if (key0 + BN - 1 > wave_minpos) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = key0 + 32 * kb + 16 * (v >> 3) + 8 * lgrp + (v & 7);
            if (key > qpos) sacc[kb][v] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kb][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx * sc);
      const float alpha = exp2f(m_run - m_new);
      float rs = 0.0f;
      u32x4 pf[2][2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = exp2f(__builtin_fmaf(sacc[kb][8 * st + 2 * w], sc, -m_new));
            const float p1 = exp2f(__builtin_fmaf(sacc[kb][8 * st + 2 * w + 1], sc, -m_new));
            rs += p0 + p1;
            pf[kb][st][w] = pack_f16x2(p0, p1);
          }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int x = 0; x < NDB; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[x][e] *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = db * 32 + lrow;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int ch = 4 * kb + 2 * st + lgrp;
            const u32x4 vf = *reinterpret_cast<const u32x4*>(sv + row * 128 + ((ch ^ (row & 7)) << 4));
            oacc[db] = mfma_f16(vf, pf[kb][st], oacc[db]);
          }
      }
    }
    if (kt + 1 < nkt) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store ------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (wave_active && lane_valid) {
    const float inv = 1.0f / l_tot;
    uint16_t* orow = a.o + ((int64_t)b * s.T + t_lane) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = db * 32 + 8 * q4 + 4 * lgrp;
        u32x2 pk{pack_f16x2(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv),
                 pack_f16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + d) = pk;
      }
  }
}

hipError_t launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* knat,
                             const uint16_t* vnat, uint16_t* o, hipStream_t st) {
  AttnArgs a;
  a.q = q;
  a.knat = knat;
  a.vnat = vnat;
  a.o = o;
  a.s = s;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s.dh));
  a.nrb = (s.c + 127) / 128;
  dim3 grid((unsigned)(2 * a.nrb * s.B * s.Hq));
  if (s.dh == 128)
    hipLaunchKernelGGL(flash_attn_kernel<128>, grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(flash_attn_kernel<64>, grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tsp
