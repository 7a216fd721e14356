// Causal flash attention of one rank's queries over the natural-order K/V
// (gfx950, f16 matrix cores, float32 online softmax).
//
// Zyphra TSP article on ai-trends.today, section "How to Fold a Book": after
// the all-gather and the zigzag reorder, every rank runs attention of its own
// tokens against the whole K/V context.  Blockwise attention keeps a running
// row maximum and row sum and rescales the partial output when the maximum
// grows (r007.github.io "Распределенное обучение", section "Параллелизм по
// контексту: Ring Attention против Ulysses": the online-softmax accumulator),
// so the S x S score matrix is never stored.
//
// Work: a block is 32 x (waves per block) consecutive local rows of one
// half of the rank's rows (a zigzag chunk, or half of the striped rows) for
// one (sequence, q-head), 32 query rows per wave; its waves share every K/V
// tile loaded into LDS.  With zigzag the later chunk sees a key prefix up to
// 2D-1 times longer than the earlier one, so a block whose key range exceeds
// kt_max tiles of 64 keys is cut into pieces along the keys (each piece keeps
// its own max / sum / unnormalised output, merged afterwards in piece order,
// so results are deterministic).  Units are ordered heaviest block first;
// when blocks are cut, each later-half block and its earlier-half partner
// share units: their combined key range is cut into equal pieces
// (block_geo), so the units weigh about the same.
//
// Per 64-key tile:
//   S^T = K Q^T   (32x32x16 MFMA, K from LDS as the first operand, the wave's
//                  Q rows kept in registers as the second) -> each lane holds
//                  one query (column) and 32 of the tile's 64 keys; the lane
//                  pair (l, l^32) shares a query, so row max/sum need only one
//                  cross-half exchange.
//   K rows are stored in LDS in a permuted order so that, for every 16-key
//   step of the P V product, a lane's 8 probabilities are 8 consecutive keys;
//   V is stored key-major, as it arrives, and read with the transposing LDS
//   load (ds_read_b64_tr_b16: 16 lanes that each point at 4 head-dim values
//   of one key row receive, per lane, 4 consecutive keys of one head-dim
//   column), two of which give a lane its 8 keys.
//   O^T += V^T P  (32x32x16 MFMA, probabilities rounded to f16).
// K and V tiles are copied global -> LDS with 16-byte direct loads into an
// NST-deep ring, straight from the all-gathered K/V slots: the partition's
// map (zigzag: position p -> chunk p / c -> source rank and local row;
// striped: rank p mod D, row p div D) is applied to the row addresses, so no
// reordered copy of K/V is made.  The barrier between
// tiles carries no memory fence, so the loads of later tiles stay in flight
// across it.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "attn_plan.h"
#include "common.h"
#include "kernels.h"

namespace tsp {

struct AttnArgs {
  const uint16_t* q;     // f16 [B][Hq][T][dh]
  const uint16_t* kv;    // f16 all-gathered K/V [D shard][D src][K|V][B][T][Hkv/D * dh]
  uint16_t* o;           // f16 [B][T][Hq*dh]
  float* part_o;         // f16 [pieces][B*Hq][rb][dh] outputs of split blocks, each piece's
                         // normalised by its own sum (float-sized slots, half used)
  float* part_ml;        // [pieces][B*Hq][2][rb] (scaled max, sum)
  float* lse;            // optional [B][Hq][T]: log2 of each row's softmax normaliser
                         // (scaled scores), so that p = 2^(s * scale_log2 - lse)
  MergeTab mtab;         // the split blocks, for the merge
  Shape s;
  float scale_log2;      // log2(e) / sqrt(dh)
  int32_t rb;            // rows per block: 32 per wave (128 or 256)
  int32_t nrb;           // row blocks per chunk
  int32_t kt_max;        // key tiles per piece at most
  int32_t pair;          // 1: each earlier-chunk block rides with a later-chunk block
};

// Row permutation inside each 32-key group: swaps 4-row blocks 1<->2, 5<->6.
__device__ __forceinline__ int key_perm(int i) {
  const int b4 = (i >> 2) & 7;
  return ((b4 ^ (b4 >> 1)) & 1) ? (i ^ 12) : i;
}

// 16-byte LDS accesses are served 16 lanes at a time over 64 four-byte banks.
// K rows are DH*2 bytes: with 256-byte rows every row starts at bank 0, so
// slot c of row r sits at c ^ (r & 15); with 128-byte rows (and the 128-byte
// rows of the transposed V tile) rows alternate bank halves, so the XOR key is
// (r >> 1) & 7.  Either way the 16 rows of one operand read hit 16 distinct
// bank groups.
template <int DH>
__device__ __forceinline__ int kswz(int row) {
  return DH == 128 ? (row & 15) : ((row >> 1) & 7);
}
// Key-major V rows are DH*2 bytes = DH/32 64-byte chunks.  A transposing PV
// read touches one 64-byte chunk of 4 consecutive key rows per 32 lanes; the
// chunk index is XORed with the row so those 4 rows sit in 4 different
// 64-byte bank windows.
template <int DH>
__device__ __forceinline__ int vswz(int row) {
  return DH == 128 ? (row & 3) : ((row >> 1) & 1);
}

// max / sum over a lane and its partner lane ^ 32: v_permlane32_swap on two
// copies of x leaves {x_l, x_(l^32)} in the two results of every lane
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


// K/V tile addressing (KM):
//   KM_ROW    any shape: every lane maps its own key through gathered_row;
//   KM_CHUNK  zigzag with chunks a whole multiple of 64 keys: a key tile
//             never straddles two chunks, so its gathered rows are
//             consecutive (one address per tile, fixed lane offsets);
//   KM_STRIPE striped with D dividing 64 and S a multiple of 64: key
//             key0 + k sits on rank k mod D (key0 is a multiple of D) at row
//             key0 / D + k div D, so every lane keeps a fixed offset from the
//             tile's row key0 / D of rank 0.
enum { KM_ROW = 0, KM_CHUNK = 1, KM_STRIPE = 2 };

// NWV waves per block (block rows 32 NWV), NST-deep LDS ring of K/V tiles.
template <int DH, int NST, int KM, int NWV>
__global__ __launch_bounds__(64 * NWV, NWV == 4 && NST == 2 ? 2 : 1) void flash_attn_kernel(AttnArgs a) {
  constexpr int BN = 64;
  constexpr int KROW = DH * 2;
  constexpr int K_BYTES = BN * KROW;
  constexpr int V_BYTES = BN * KROW;
  constexpr int STAGE = K_BYTES + V_BYTES;
  constexpr int KRPI = 1024 / KROW;          // K (and V) rows per direct-load instruction
  constexpr int K_INS = BN / KRPI;           // instructions per K tile
  constexpr int V_INS = BN / KRPI;           // ... per V tile
  constexpr int QT = K_INS + V_INS;
  static_assert(QT % NWV == 0, "loads split evenly over the waves");
  constexpr int QW = QT / NWV;               // per wave
  constexpr int RBR = 32 * NWV;              // rows per block
  constexpr int NDB = DH / 32;
  constexpr int NKS = DH / 16;
  __shared__ __align__(16) unsigned char smem[NST * STAGE];

  const Shape& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  // transposing V reads: lane (group gq = lane / 16, s = lane % 16) points at
  // key row 8 (gq / 2) + s / 4 (+ the step's key base) and head-dim columns
  // db * 32 + 16 (gq % 2) + 4 (s % 4) .. + 3
  int vlane[NDB];
  {
    const int gq = lane >> 4, sl = lane & 15;
    const int vrow = 8 * (gq >> 1) + (sl >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      vlane[db] = vrow * KROW + ((db ^ vswz<DH>(vrow)) << 6) + 32 * (gq & 1) + 8 * (sl & 3);
  }

  // ---- work unit -> (block, piece, sequence, q-head) --------------------
  const int per_bh = s.B * s.Hq;
  const PlanKey pk{s.c, s.D, s.r, s.part, RBR, a.nrb, a.kt_max, a.pair};
  const UnitPos up = unit_of(pk, per_bh, blockIdx.x);
  const int piece = up.piece, bh = up.bh, piece_base = up.piece_base;
  const int b = bh / s.Hq, qh = bh - b * s.Hq;
  // paired plan: the unit's piece of the pair's combined key range may also
  // (or only) cover tiles of the earlier-half partner block
  const PieceSplit psp = piece_split(pk, up.g, up.bi);

  const int G = qh / (s.Hq / s.Hkv);
  const int jsh = G / s.Hkv_s, hk = G - jsh * s.Hkv_s;
  const int kvd = s.Hkv_s * DH;
  const int64_t head_off = (int64_t)hk * DH;
  const int64_t v_step = (int64_t)s.B * s.T * kvd;  // K slot -> V slot of the same rows

  // ---- direct-load assignment: wave instruction q = wave + NWV i ----------
  // K rows go to LDS in permuted order with XOR-swizzled 16-byte slots; V
  // rows in natural order with XOR-swizzled 64-byte chunks.
  int lkey[QW], lcol[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + NWV * i;
    const int slot = lane % (KROW / 16);
    if (q < K_INS) {
      const int row = KRPI * q + lane / (KROW / 16);
      lkey[i] = (row & ~31) | key_perm(row & 31);
      lcol[i] = (slot ^ kswz<DH>(row)) * 8;
    } else {
      const int row = KRPI * (q - K_INS) + lane / (KROW / 16);
      lkey[i] = row;
      lcol[i] = (4 * ((slot >> 2) ^ vswz<DH>(row)) + (slot & 3)) * 8;
    }
  }
  // KM_CHUNK / KM_STRIPE: byte offset of each lane's 16 bytes from the
  // tile's base row (V rows sit v_step elements further), the same for every
  // tile; the host checks that they fit in 31 bits.  KM_CHUNK: the tile
  // cursor (chunk kq, key kr within it) advances by one tile per issue, as
  // issue() is called for consecutive tiles.
  const int64_t src_step = 2 * v_step;  // rank src -> src + 1, same rows
  uint32_t loff[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int q = wave + NWV * i;
    const int64_t row_off = KM == KM_STRIPE ? (int64_t)(lkey[i] % s.D) * src_step + (int64_t)(lkey[i] / s.D) * kvd
                                            : (int64_t)lkey[i] * kvd;
    loff[i] = (uint32_t)(((q < K_INS ? 0 : v_step) + row_off + lcol[i]) * 2);
  }

  for (int part = 0; part < (a.pair ? 2 : 1); ++part) {
    // split: this piece's partial state goes to workspace slot piece_base +
    // slot for the merge
    BlockGeo g;
    int kt_begin, kt_end, slot;
    bool split;
    if (!unit_part(pk, up.g, up.bi, psp, piece, part, g, kt_begin, kt_end, split, slot)) continue;
    const int wt0 = g.t0 + wave * 32;
    const bool wave_active = wt0 < g.row_end;
    int t_lane = wt0 + lrow;
    const bool lane_valid = t_lane < g.row_end;
    t_lane = lane_valid ? t_lane : g.row_end - 1;
    const int qpos = g.gstart + (t_lane - g.row_begin) * g.pstride;
    const int w_last = (wt0 + 31 < g.row_end ? wt0 + 31 : g.row_end - 1);
    const int wave_maxpos = g.gstart + (w_last - g.row_begin) * g.pstride;
    const int wave_minpos = g.gstart + (wt0 - g.row_begin) * g.pstride;

    // ---- Q fragments (second operand of S^T = K Q^T) ---------------------
    u32x4 qf[NKS];
    {
      const uint16_t* qrow = a.q + (((int64_t)b * s.Hq + qh) * s.T + t_lane) * DH;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) qf[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + lgrp * 8);
    }

    int kq = (kt_begin * BN) / s.c, kr = kt_begin * BN - kq * s.c;
    auto issue = [&](int kt, int stage) {
      unsigned char* sb = smem + stage * STAGE;
      const int key0 = kt * BN;
      if constexpr (KM == KM_STRIPE) {
        const int64_t row0 = ((int64_t)jsh * s.D * 2 * s.B + b) * s.T + key0 / s.D;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.kv + row0 * kvd + head_off), (short)0, 0x7fffffff, 0x00020000);
#pragma unroll
        for (int i = 0; i < QW; ++i) {
          const int q = wave + NWV * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(sb + q * 1024), 16, (int)loff[i], 0, 0, 0);
        }
      } else if constexpr (KM == KM_CHUNK) {
        const int g_src = kq < s.D ? kq : 2 * s.D - 1 - kq;
        const int t = (kq < s.D ? 0 : s.c) + kr;
        const int64_t row0 = ((((int64_t)jsh * s.D + g_src) * 2) * s.B + b) * s.T + t;
        const __amdgpu_buffer_rsrc_t rsrc =
            __builtin_amdgcn_make_buffer_rsrc((void*)(a.kv + row0 * kvd + head_off), (short)0, 0x7fffffff, 0x00020000);
        kr += BN;
        if (kr >= s.c) {
          kr -= s.c;
          ++kq;
        }
#pragma unroll
        for (int i = 0; i < QW; ++i) {
          const int q = wave + NWV * i;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(sb + q * 1024), 16, (int)loff[i], 0, 0, 0);
        }
        (void)key0;
      } else {
#pragma unroll
        for (int i = 0; i < QW; ++i) {
          const int q = wave + NWV * i;
          int p = key0 + lkey[i];
          p = p < s.S ? p : s.S - 1;  // keys past the sequence end are masked
          const int64_t off = gathered_row(s, jsh, q < K_INS ? 0 : 1, b, p) * kvd + head_off + lcol[i];
          attn_load_lds16(a.kv + off, sb + q * 1024);
        }
      }
    };
    auto wait_tile = [&](int newer) {  // loads of later tiles may stay in flight
      if constexpr (NST >= 3) {
        if (newer >= 1) {
          __builtin_amdgcn_s_waitcnt((QW & 15) | ((QW >> 4) << 14) | (7 << 4) | (0 << 8));
          return;
        }
      }
      __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8));
    };
    auto barrier = [&]() {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int x = 0; x < NDB; ++x)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[x][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const float sc = a.scale_log2;

    // ---- the three parts of one key tile ----------------------------------
    // S^T = K Q^T with K at sk
    auto s_block = [&](const unsigned char* sk, f32x16 (&sacc)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < 2; ++x)
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[x][e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int pch = ((2 * ks + lgrp) ^ kswz<DH>(lrow)) << 4;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 kf = *reinterpret_cast<const u32x4*>(sk + (kb * 32 + lrow) * KROW + pch);
          sacc[kb] = mfma_f16(kf, qf[ks], sacc[kb]);
        }
      }
    };
    // causal mask and online softmax of the tile at key0: probabilities to
    // pf (f16), running max / sum updated, O rescaled when the max moved
    auto softmax_block = [&](int key0, f32x16 (&sacc)[2], u32x4 (&pf)[2][2]) __attribute__((always_inline)) {
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
      mx = pair_max(mx);
      // The reference maximum m_run moves only when the row maximum passes it
      // by more than 8 (log2 units).  Exponents then stay <= 8 (probabilities
      // < 256: fine for f16 P and the float32 sums), numerator and denominator
      // share the reference so the result is the same, and most tiles skip
      // the rescale of O.
      const float m_max = fmaxf(m_run, mx * sc);
      const float m_new = m_max > m_run + 8.0f ? m_max : m_run;
      // a row with no unmasked key yet keeps m = -inf; its probabilities are 0
      const float m_sub = m_new == -INFINITY ? 0.0f : m_new;
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * st + 2 * w], sc, -m_sub));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * st + 2 * w + 1], sc, -m_sub));
            const uint32_t pk = pack_f16x2(p0, p1);
            pf[kb][st][w] = pk;
            // the row sum is taken over the f16 probabilities that P V uses
            rs = __builtin_amdgcn_fdot2(__builtin_bit_cast(__attribute__((ext_vector_type(2))) _Float16, pk),
                                        (__attribute__((ext_vector_type(2))) _Float16){1.0f16, 1.0f16}, rs, false);
          }
      // rescale only when some row's maximum moved (alpha == 1 otherwise)
      if (__any(m_new != m_run)) {
        const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int x = 0; x < NDB; ++x)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[x][e] *= alpha;
      }
      l_run += rs;
      m_run = m_new;
    };
    // O^T += V^T P with V at sv
    auto pv_block = [&](const unsigned char* sv, const u32x4 (&pf)[2][2]) __attribute__((always_inline)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            // keys 32 kb + 16 st + 8 (lane / 32) + 4 r + (0..3), head-dim column db * 32 + lane % 32
            const unsigned char* vp = sv + vlane[db] + (32 * kb + 16 * st) * KROW;
            const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)vp);
            const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(vp + 4 * KROW));
            const u32x2 h0 = __builtin_bit_cast(u32x2, r0), h1 = __builtin_bit_cast(u32x2, r1);
            const u32x4 vf{h0[0], h0[1], h1[0], h1[1]};
            oacc[db] = mfma_f16(vf, pf[kb][st], oacc[db]);
          }
      }
    };

    {
      int issued = 0;
#pragma unroll
      for (int i = 0; i < NST - 1; ++i)
        if (kt_begin + i < kt_end) {
          issue(kt_begin + i, i);
          ++issued;
        }
      wait_tile(issued - 1);
      barrier();
    }
    // one key tile; the LDS stage is a compile-time constant so that every
    // LDS address is a per-lane base plus an immediate
    auto step = [&](int kt, auto ST_) __attribute__((always_inline)) {
      constexpr int stage = decltype(ST_)::value;
      constexpr int fill = (stage + NST - 1) % NST;
      if (kt + NST - 1 < kt_end) issue(kt + NST - 1, fill);
      const int key0 = kt * BN;
      if (wave_active && key0 <= wave_maxpos) {
        const unsigned char* sk = smem + stage * STAGE;
        f32x16 sacc[2];
        u32x4 pf[2][2];
        s_block(sk, sacc);
        softmax_block(key0, sacc, pf);
        pv_block(sk + K_BYTES, pf);
      }
      const int last_issued = (kt + NST - 1 < kt_end) ? kt + NST - 1 : kt_end - 1;
      wait_tile(last_issued - (kt + 1));
      barrier();
    };
    // tile kt_begin + j sits in stage j mod NST
    int kt = kt_begin;
    for (; kt + NST - 1 < kt_end; kt += NST)
      static_for<0, NST>([&](auto I) __attribute__((always_inline)) { step(kt + decltype(I)::value, I); });
    static_for<0, NST - 1>([&](auto I) __attribute__((always_inline)) {
      if (kt + decltype(I)::value < kt_end) step(kt + decltype(I)::value, I);
    });

    // ---- store: final f16 output, or the piece's partial state ------------
    const float l_tot = pair_sum(l_run);
    if (!wave_active || !lane_valid) continue;
    if (!split) {
      const float inv = 1.0f / l_tot;
      if (a.lse != nullptr && lgrp == 0) a.lse[((int64_t)b * s.Hq + qh) * s.T + t_lane] = m_run + log2f(l_tot);
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
    } else {
      const int64_t pidx = (int64_t)(piece_base + slot) * per_bh + bh;
      const int r = t_lane - g.t0;
      // the piece's output normalised by its own sum (|.| <= max |v|: f16
      // holds it whatever the piece's length); the merge weights it back.  A
      // row whose keys in this piece are all masked has sum 0 and weight 0:
      // it stores zeros (not 0 / 0)
      uint16_t* po = reinterpret_cast<uint16_t*>(a.part_o) + (pidx * RBR + r) * DH;
      const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int d = db * 32 + 8 * q4 + 4 * lgrp;
          u32x2 pk{pack_f16x2(oacc[db][4 * q4] * inv, oacc[db][4 * q4 + 1] * inv),
                   pack_f16x2(oacc[db][4 * q4 + 2] * inv, oacc[db][4 * q4 + 3] * inv)};
          *reinterpret_cast<u32x2*>(po + d) = pk;
        }
      if (lgrp == 0) {
        a.part_ml[(pidx * 2 + 0) * RBR + r] = m_run;
        a.part_ml[(pidx * 2 + 1) * RBR + r] = l_tot;
      }
    }
  }
}

// Combines the pieces of every split block, in piece order:
// O = sum_p w_p Ô_p / sum_p w_p, w_p = 2^(m_p - m) l_p, m = max_p m_p, with
// Ô_p = O_p / l_p the piece's normalised output.  One thread per (row, 4
// head-dim columns).  A split block holds B Hq rb DH / 4 items, a multiple of
// the 256-thread work group, so the block is located from the work group's
// first item (the same for every lane), through the host's table of split
// blocks.
template <int DH>
__global__ void attn_merge_kernel(AttnArgs a) {
  const Shape& s = a.s;
  const int per_bh = s.B * s.Hq;
  constexpr int cols = DH / 4;
  const long long ipb = (long long)per_bh * a.rb * cols;  // items per split block
  // locate the split block this work group belongs to: from the host's
  // table, or by walking the plan when the table could not hold it
  BlockGeo g;
  int piece_base, npieces;
  long long item0;
  if (a.mtab.n >= 0) {
    const long long first = (long long)blockIdx.x * blockDim.x;
    const int e = (int)(first / ipb);
    if (e >= a.mtab.n) return;
    g = block_rows(s.c, s.D, s.r, s.part, a.rb, a.nrb, a.mtab.bi[e]);
    piece_base = a.mtab.base[e];
    npieces = a.mtab.np[e];
    item0 = first - (long long)e * ipb;
  } else {
    const PlanKey plan{s.c, s.D, s.r, s.part, a.rb, a.nrb, a.kt_max, a.pair};
    const MergePos mp = merge_block_of(plan, ipb, (long long)blockIdx.x * blockDim.x);
    if (mp.bi < 0) return;
    g = mp.g;
    piece_base = mp.piece_base;
    npieces = mp.npieces;
    item0 = mp.item;
  }
  const int64_t item = item0 + threadIdx.x;
  const int c4 = (int)(item % cols);
  const int r = (int)((item / cols) % a.rb);
  const int bh = (int)(item / (cols * a.rb));
  const int t = g.t0 + r;
  if (t >= g.row_end) return;
  float mmax = -INFINITY;
  for (int p = 0; p < npieces; ++p) {
    const int64_t pidx = (int64_t)(piece_base + p) * per_bh + bh;
    mmax = fmaxf(mmax, a.part_ml[(pidx * 2 + 0) * a.rb + r]);
  }
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  float l = 0.f;
  for (int p = 0; p < npieces; ++p) {
    const int64_t pidx = (int64_t)(piece_base + p) * per_bh + bh;
    // weight of the piece: 2^(m_p - m) l_p, its output stored normalised
    const float w = __builtin_amdgcn_exp2f(a.part_ml[(pidx * 2 + 0) * a.rb + r] - mmax) *
                    a.part_ml[(pidx * 2 + 1) * a.rb + r];
    l += w;
    const u32x2 v = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint16_t*>(a.part_o) +
                                                    (pidx * a.rb + r) * DH + 4 * c4);
    const uint32_t v0 = v[0], v1 = v[1];
    const f16x2 h0 = __builtin_bit_cast(f16x2, v0), h1 = __builtin_bit_cast(f16x2, v1);
    acc[0] += w * (float)h0[0];
    acc[1] += w * (float)h0[1];
    acc[2] += w * (float)h1[0];
    acc[3] += w * (float)h1[1];
  }
  const float inv = 1.0f / l;
  const int b = bh / s.Hq, qh = bh - b * s.Hq;
  if (a.lse != nullptr && c4 == 0) a.lse[((int64_t)b * s.Hq + qh) * s.T + t] = mmax + log2f(l);
  uint16_t* orow = a.o + ((int64_t)b * s.T + t) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH + 4 * c4;
  u32x2 pk{pack_f16x2(acc[0] * inv, acc[1] * inv), pack_f16x2(acc[2] * inv, acc[3] * inv)};
  *reinterpret_cast<u32x2*>(orow) = pk;
}

// ---- host-side plan (shared with workspace sizing) -----------------------
// Kernel shape: waves per block (32 rows each) and depth of the K/V ring.
// 4 waves and 2 stages fit two blocks per CU; 8 waves and 3 stages run one
// block per CU, each K/V tile shared by 256 query rows (half the K/V
// traffic).  The second pays off only when blocks loop over long key ranges
// (measured: 3% faster at 128K context with ~1100 key tiles per block, 2-5%
// slower at 130-260), so it is taken when the rank's 128-row blocks average
// at least 512 key tiles.  Override (tsp_set_tuning, TSP_TUNE_ATTN_SHAPE):
// 4 or 8 waves.
struct AttnShape {
  int nwv, nst;
};
static const AttnShape kShapes[] = {{4, 2}, {8, 3}};
enum { KNOB_ATTN_SHAPE = 6, KNOB_ATTN_PAIR = 7, KNOB_ATTN_PIECES = 8 };

static AttnShape attn_shape(const Shape& s) {
  const int over = tune_get(KNOB_ATTN_SHAPE);
  for (const AttnShape& k : kShapes)
    if (over == k.nwv) return k;
  const int rbr = 32 * kShapes[0].nwv, nrb = (s.c + rbr - 1) / rbr;
  long long tiles = 0;
  for (int bi = 0; bi < 2 * nrb; ++bi) tiles += block_rows(s.c, s.D, s.r, s.part, rbr, nrb, bi).nkt;
  return tiles >= 512LL * 2 * nrb ? kShapes[1] : kShapes[0];
}

// Estimated finishing time of a plan, in key tiles: units are handed out in
// launch order to the first of `slots` resident work groups to become free;
// a unit costs its key tiles plus kUnitCost (loading Q, writing the output
// or the partial state, the merge).
static long long plan_makespan(const PlanKey& k, int per_bh, long long slots) {
  constexpr int kUnitCost = 2;
  // min-heap of the resident work groups' finishing times (at most 512 of
  // them: a fixed array, so planning allocates nothing)
  constexpr int kMaxSlots = 512;
  long long heap[kMaxSlots];
  const int n = (int)(slots < kMaxSlots ? slots : kMaxSlots);
  for (int i = 0; i < n; ++i) heap[i] = 0;
  const auto later = [](long long x, long long y) { return x > y; };
  long long end = 0;
  for (int bi = 0; bi < 2 * k.nrb; ++bi) {
    const BlockGeo g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, bi);
    const PieceSplit sp = piece_split(k, g, bi);
    for (int p = 0; p < g.ns; ++p) {
      int w = kUnitCost;
      for (int which = 0; which < 2; ++which) {
        BlockGeo pg;
        int kb, ke, slot;
        bool split;
        if (unit_part(k, g, bi, sp, p, which, pg, kb, ke, split, slot)) w += ke - kb;
      }
      for (int bh = 0; bh < per_bh; ++bh) {
        std::pop_heap(heap, heap + n, later);       // earliest-free work group to the back
        heap[n - 1] += w;
        end = heap[n - 1] > end ? heap[n - 1] : end;
        std::push_heap(heap, heap + n, later);
      }
    }
  }
  return end;
}

// pair < 0: the default.  Blocks are split when there are fewer than twice
// as many as resident work groups; pieces then hold about tiles / (resident
// work groups) key tiles, and the earlier half's blocks ride with the later
// half's (paired) unless the makespan estimate says that separate units
// finish sooner (when both halves see long key ranges: zigzag on the middle
// and last ranks, striped).  Overrides (tsp_set_tuning): TSP_TUNE_ATTN_PIECES
// = target number of work units, TSP_TUNE_ATTN_PAIR = 0 or 1.
static AttnPlan plan_for(const Shape& s, int pair, AttnShape k) {
  AttnPlan p;
  p.nwv = k.nwv;
  p.nst = k.nst;
  p.rb = 32 * k.nwv;
  const long long slots = k.nwv == 4 && k.nst == 2 ? 512 : 256;  // resident blocks on 256 CUs
  long long target = slots;
  if (tune_get(KNOB_ATTN_PIECES) > 0) target = tune_get(KNOB_ATTN_PIECES);
  if (pair < 0) {
    const int over = tune_get(KNOB_ATTN_PAIR);
    if (over == 0 || over == 1) {
      pair = over;
    } else {
      const PlanKey kp = plan_key(s.c, s.D, s.r, s.part, s.B, s.Hq, p.rb, slots, target, 1);
      pair = 1;
      if (kp.pair) {
        const PlanKey ku = plan_key(s.c, s.D, s.r, s.part, s.B, s.Hq, p.rb, slots, target, 0);
        if (plan_makespan(ku, s.B * s.Hq, slots) < plan_makespan(kp, s.B * s.Hq, slots)) pair = 0;
      }
    }
  }
  const PlanKey key = plan_key(s.c, s.D, s.r, s.part, s.B, s.Hq, p.rb, slots, target, pair);
  const PlanCounts n = plan_counts(key);
  p.nrb = key.nrb;
  p.kt_max = key.kt_max;
  p.pair = key.pair;
  p.units = n.units_per_bh * s.B * s.Hq;
  p.pieces = n.pieces;
  p.split_rows = n.split_rows;
  return p;
}

// The plan is recomputed on every launch (no state is kept between calls);
// its cost is a few thousand integer steps at most, and only shapes whose
// blocks are split along the keys estimate the makespan at all.
AttnPlan attn_plan(const Shape& s) { return plan_for(s, -1, attn_shape(s)); }

AttnPlan attn_plan_shape(const Shape& s, int nwv) {
  for (const AttnShape& k : kShapes)
    if (k.nwv == nwv) return plan_for(s, -1, k);
  return plan_for(s, -1, kShapes[0]);
}

// Enough for every plan, so that a workspace sized once serves them all.
size_t attn_partial_bytes(const Shape& s) {
  size_t most = 0;
  for (const AttnShape& k : kShapes)
    for (int pair = 0; pair < 2; ++pair) {
      const AttnPlan p = plan_for(s, pair, k);
      const size_t b = (size_t)p.pieces * s.B * s.Hq * p.rb * (s.dh + 2) * sizeof(float);
      most = b > most ? b : most;
    }
  return most;
}

template <int DH, int NST, int NWV>
static void launch_fa(const AttnArgs& a, int km, unsigned units, hipStream_t st) {
  if (km == KM_CHUNK)
    hipLaunchKernelGGL((flash_attn_kernel<DH, NST, KM_CHUNK, NWV>), dim3(units), dim3(64 * NWV), 0, st, a);
  else if (km == KM_STRIPE)
    hipLaunchKernelGGL((flash_attn_kernel<DH, NST, KM_STRIPE, NWV>), dim3(units), dim3(64 * NWV), 0, st, a);
  else
    hipLaunchKernelGGL((flash_attn_kernel<DH, NST, KM_ROW, NWV>), dim3(units), dim3(64 * NWV), 0, st, a);
}

template <int DH>
static void launch_fa_shape(const AttnPlan& p, const AttnArgs& a, int km, hipStream_t st) {
  const unsigned units = (unsigned)p.units;
  if (p.nwv == 4)
    launch_fa<DH, 2, 4>(a, km, units, st);
  else
    launch_fa<DH, 3, 8>(a, km, units, st);
}

hipError_t launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* kv_gathered, uint16_t* o,
                             float* partial, hipStream_t st, float* lse) {
  const AttnPlan p = attn_plan(s);
  AttnArgs a;
  a.lse = lse;
  a.q = q;
  a.kv = kv_gathered;
  a.o = o;
  a.part_o = partial;
  a.part_ml = partial + (size_t)p.pieces * s.B * s.Hq * p.rb * s.dh;
  a.s = s;
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s.dh));
  a.rb = p.rb;
  a.nrb = p.nrb;
  a.kt_max = p.kt_max;
  a.pair = p.pair;
  a.mtab = merge_table(PlanKey{s.c, s.D, s.r, s.part, p.rb, p.nrb, p.kt_max, p.pair});
  // the whole-tile paths address a tile's K and V rows with 31-bit offsets
  // (the largest: the V row of the last key, from the tile's base row)
  const int64_t kvd = (int64_t)s.Hkv_s * s.dh;
  const int64_t v_step = (int64_t)s.B * s.T * kvd;
  int km = KM_ROW;
  if (s.part == 0 && s.c % 64 == 0 && (v_step + 64 * kvd) * 2 < ((int64_t)1 << 31)) km = KM_CHUNK;
  if (s.part == 1 && 64 % s.D == 0 && s.S % 64 == 0 &&
      (v_step + (int64_t)(s.D - 1) * 2 * v_step + (64 / s.D) * kvd) * 2 < ((int64_t)1 << 31))
    km = KM_STRIPE;
  if (s.dh == 128)
    launch_fa_shape<128>(p, a, km, st);
  else
    launch_fa_shape<64>(p, a, km, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.pieces == 0) return e;
  const int64_t items = (int64_t)p.split_rows * s.B * s.Hq * (s.dh / 4);
  const unsigned blocks = (unsigned)((items + 255) / 256);
  if (s.dh == 128)
    hipLaunchKernelGGL(attn_merge_kernel<128>, dim3(blocks), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(attn_merge_kernel<64>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace tsp
