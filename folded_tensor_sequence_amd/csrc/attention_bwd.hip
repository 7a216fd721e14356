// Backward of the causal attention of one rank's queries (gfx950, f16 matrix
// cores, float32 accumulation and softmax).
//
// The pages give TSP's forward schedule only (Zyphra TSP article on
// ai-trends.today, section "How to Fold a Book": each rank attends with its
// own queries over the all-gathered K/V of every rank).  Its backward is the
// transpose: the rank differentiates its own queries' attention over all
// keys; the query gradient stays local, and the gradients this produces for
// every key's K and V rows are reduce-scattered to the ranks owning those
// keys.  With the softmax normaliser L of each row kept from the forward
// (lse, log2 units of the scaled scores), for one head:
//
//   P  = 2^(S sc - L)            S = Q K^T, sc = log2(e) / sqrt(dh)
//   dP = dO V^T,  Delta = rowsum(dO * O),  dS = P * (dP - Delta)
//   dQ = dS K / sqrt(dh),  dK = dS^T Q / sqrt(dh),  dV = P^T dO
//
// (the online-softmax form of r007.github.io "Распределенное обучение",
// section "Параллелизм по контексту: Ring Attention против Ulysses", run
// backwards with the normaliser known, so blocks of keys are independent).
//
// Two kernels, so that every gradient is a plain sum with a fixed order
// (no atomics, bitwise reproducible):
//   attn_bwd_dq_kernel   query-major, the forward's work plan (row blocks of
//                        128 queries, long key ranges cut into pieces whose
//                        partial dQ are summed in piece order afterwards);
//                        K/V tiles of 64 keys stream through LDS;
//   attn_bwd_dkv_kernel  key-major: a work group owns 128 keys of one
//                        (sequence, kv-head); tiles of 64 of the rank's
//                        queries (Q, dO, L, Delta; every q-head of the kv
//                        head's group) stream through LDS.
// Matrix-core operands follow the layout of mfma_f16 (common.h): a lane
// feeds row lane%32 of an operand with 8 consecutive k-values, and holds
// column lane%32, rows 8(v/4) + 4(lane/32) + v%4, of the result.  A result
// tile used as the next product's k-operand (P, dS) keeps that row order;
// the other operand of that product is read with the transposing LDS load,
// whose two halves per 16-row step cover rows {0-3, 8-11} (lanes 0-31) and
// {4-7, 12-15} (lanes 32-63), matching it.  LDS tile rows are stored in
// natural order with 16-byte slots XOR-swizzled so that both the row-wise
// operand reads and the transposing reads are free of bank conflicts.
#include <math.h>

#include "attn_common.h"
#include "attn_plan.h"
#include "common.h"
#include "kernels.h"

namespace tsp {

struct AttnBwdArgs {
  const uint16_t* q;     // f16 [B][Hq][T][dh]
  const uint16_t* kv;    // f16 all-gathered K/V [D shard][D src][K|V][B][T][Hkv/D * dh]
  const uint16_t* o;     // f16 [B][T][Hq*dh]
  const uint16_t* dout;  // f16 [B][T][Hq*dh]  (dO)
  const float* lse;      // [B][Hq][T]
  float* delta;          // [B][Hq][T]
  float* dq;             // [B][T][Hq*dh]
  float* dkv;            // [D dst][D shard][K|V][B][T][Hkv/D * dh]
  float* part;           // [pieces][B*Hq][rb][dh] partial dQ of split row blocks
  Shape s;
  float scale_log2;      // log2(e) / sqrt(dh)
  float scale;           // 1 / sqrt(dh)
  int32_t rb, nrb, kt_max, pair;  // the dQ kernel's work plan
  MergeTab mtab;                  // its split blocks, for the piece sums
};

namespace {

// Slot swizzle of a tile row: row-wise reads touch 16 consecutive rows at one
// slot (need 16 distinct bank groups); transposing reads touch 4 aligned
// consecutive rows x 64 bytes (need 4 distinct 64-byte bank windows).
// 256-byte rows (dh 128): slot ^= (row % 4) * 4 + (row / 4) % 4.  128-byte
// rows (dh 64; two rows per 256 bytes of banks): slot ^= ((row / 2) % 2) * 4
// + (row / 4) % 4.
template <int DH>
__device__ __forceinline__ int bswz(int row) {
  return DH == 128 ? (((row & 3) << 2) | ((row >> 2) & 3)) : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

// Byte offsets (within a tile, relative to its 16-row step) of the two
// transposing reads that give a lane its 8 k-values (rows) of head-dim column
// db * 32 + lane % 32: lane (group gq = lane / 16, s = lane % 16) points at
// row 4 (gq / 2) + s / 4 (+ 8 for the second read), columns db*32 + 16 (gq %
// 2) + 4 (s % 4) .. + 3.
template <int DH>
__device__ __forceinline__ int tr_offset(int lane, int db, int second) {
  constexpr int KROW = DH * 2;
  const int gq = lane >> 4, sl = lane & 15;
  const int row = 4 * (gq >> 1) + (sl >> 2) + 8 * second;
  const int c0 = db * 32 + 16 * (gq & 1) + 4 * (sl & 3);
  return row * KROW + (((c0 >> 3) ^ bswz<DH>(row)) << 4) + (c0 & 7) * 2;
}

__device__ __forceinline__ u32x4 tr_read(const unsigned char* p0, const unsigned char* p1) {
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p0);
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p1);
  const u32x2 h0 = __builtin_bit_cast(u32x2, r0), h1 = __builtin_bit_cast(u32x2, r1);
  return u32x4{h0[0], h0[1], h1[0], h1[1]};
}

__device__ __forceinline__ void barrier_nofence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt((7 << 4) | (0 << 8)); }

}  // namespace

// ---- Delta = rowsum(dO * O) per (row, q-head) --------------------------------
// DH / 8 lanes per (row, head), 8 elements (16 bytes) each.
template <int DH>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(AttnBwdArgs a) {
  constexpr int LPR = DH / 8;
  const Shape& s = a.s;
  const int64_t item = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / LPR;
  const int sub = threadIdx.x % LPR;
  const int64_t n = (int64_t)s.M * s.Hq;
  float acc = 0.0f;
  if (item < n) {
    const int64_t off = item * DH + sub * 8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(a.dout + off);
    const u32x4 y = *reinterpret_cast<const u32x4*>(a.o + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // through scalars: a bit cast of a vector element itself is not used
      const uint32_t xe = x[e], ye = y[e];
      const f16x2 xx = __builtin_bit_cast(f16x2, xe), yy = __builtin_bit_cast(f16x2, ye);
      acc += (float)xx[0] * (float)yy[0] + (float)xx[1] * (float)yy[1];
    }
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w, 64);
  if (item < n && sub == 0) {
    const int64_t m = item / s.Hq;
    const int qh = (int)(item - m * s.Hq);
    const int b = (int)(m / s.T), t = (int)(m - (int64_t)b * s.T);
    a.delta[((int64_t)b * s.Hq + qh) * s.T + t] = acc;
  }
}

// ---- dQ: query-major --------------------------------------------------------
// 4 waves x 32 query rows per block (the forward's plan); per 64-key tile a
// wave computes S^T = K Q^T and dP^T = V dO^T (keys x its queries), forms
// dS^T and accumulates dQ^T += K^T dS^T.
template <int DH>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  constexpr int NWV = 4, BN = 64, KROW = DH * 2, TILE = BN * KROW, STAGE = 2 * TILE;
  constexpr int KRPI = 1024 / KROW;  // tile rows per 16-byte direct-load instruction
  constexpr int TI = BN / KRPI;      // instructions per tile
  constexpr int QW = 2 * TI / NWV;   // K and V instructions per wave
  constexpr int RBR = 32 * NWV;
  constexpr int NDB = DH / 32, NKS = DH / 16;
  // the two stages as two arrays, named at compile time (see stage_mem)
  __shared__ __align__(16) unsigned char smem0[STAGE];
  __shared__ __align__(16) unsigned char smem1[STAGE];
  auto stage_mem = [&](auto ST_) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (decltype(ST_)::value == 0)
      return smem0;
    else
      return smem1;
  };

  const Shape& s = a.s;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int per_bh = s.B * s.Hq;
  const PlanKey pk{s.c, s.D, s.r, s.part, RBR, a.nrb, a.kt_max, a.pair};
  const UnitPos up = unit_of(pk, per_bh, blockIdx.x);
  const int piece = up.piece, bh = up.bh, piece_base = up.piece_base;
  const int b = bh / s.Hq, qh = bh - b * s.Hq;
  const PieceSplit psp = piece_split(pk, up.g, up.bi);
  const int G = qh / (s.Hq / s.Hkv);
  const int jsh = G / s.Hkv_s, hk = G - jsh * s.Hkv_s;
  const int kvd = s.Hkv_s * DH;
  const int64_t head_off = (int64_t)hk * DH;

  // direct loads: instruction i of this wave fills tile rows KRPI * (qi % TI)
  // .. of K (qi < TI) or V; lane -> (row, physical slot), loading the
  // logical slot that the swizzle puts there
  int lrow_ld[QW], lcol_ld[QW];
#pragma unroll
  for (int i = 0; i < QW; ++i) {
    const int qi = wave + NWV * i;
    const int row = KRPI * (qi % TI) + lane / (KROW / 16);
    lrow_ld[i] = row;
    lcol_ld[i] = ((lane % (KROW / 16)) ^ bswz<DH>(row)) * 8;
  }
  int tro[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tro[db][0] = tr_offset<DH>(lane, db, 0);
    tro[db][1] = tr_offset<DH>(lane, db, 1);
  }
  const int fl = bswz<DH>(lrow);

  for (int part = 0; part < (a.pair ? 2 : 1); ++part) {
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

    // the lane's query: Q and dO rows as the k-operand of S^T and dP^T
    u32x4 qf[NKS], dof[NKS];
    {
      const uint16_t* qrow = a.q + (((int64_t)b * s.Hq + qh) * s.T + t_lane) * DH;
      const uint16_t* drow = a.dout + ((int64_t)b * s.T + t_lane) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        qf[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16 + lgrp * 8);
        dof[ks] = *reinterpret_cast<const u32x4*>(drow + ks * 16 + lgrp * 8);
      }
    }
    const int64_t rowix = ((int64_t)b * s.Hq + qh) * s.T + t_lane;
    const float lse_q = a.lse[rowix];
    const float delta_q = a.delta[rowix];

    auto issue = [&](int kt, auto ST_) __attribute__((always_inline)) {
      unsigned char* sb = stage_mem(ST_);
#pragma unroll
      for (int i = 0; i < QW; ++i) {
        const int qi = wave + NWV * i;
        const int sel = qi < TI ? 0 : 1;
        int p = kt * BN + lrow_ld[i];
        p = p < s.S ? p : s.S - 1;  // keys past the sequence end are masked
        const int64_t off = gathered_row(s, jsh, sel, b, p) * kvd + head_off + lcol_ld[i];
        attn_load_lds16(a.kv + off, sb + qi * 1024);
      }
    };

    f32x16 dqacc[NDB];
#pragma unroll
    for (int x = 0; x < NDB; ++x)
#pragma unroll
      for (int e = 0; e < 16; ++e) dqacc[x][e] = 0.0f;
    const float sc = a.scale_log2;

    if (kt_begin < kt_end) issue(kt_begin, IC<0>{});
    wait_loads();
    barrier_nofence();
    // tile kt_begin + j sits in stage j mod 2
    auto step = [&](int kt, auto ST_) __attribute__((always_inline)) {
      if (kt + 1 < kt_end) issue(kt + 1, IC<decltype(ST_)::value ^ 1>{});
      const int key0 = kt * BN;
      if (wave_active && key0 <= wave_maxpos) {
        const unsigned char* sk = stage_mem(ST_);
        const unsigned char* sv = sk + TILE;
        const bool masked = key0 + BN - 1 > wave_minpos;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          f32x16 sacc, dpacc;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            sacc[e] = 0.0f;
            dpacc[e] = 0.0f;
          }
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int off = (kb * 32 + lrow) * KROW + (((2 * ks + lgrp) ^ fl) << 4);
            sacc = mfma_f16(*reinterpret_cast<const u32x4*>(sk + off), qf[ks], sacc);
            dpacc = mfma_f16(*reinterpret_cast<const u32x4*>(sv + off), dof[ks], dpacc);
          }
          // causal edge: scores of keys after the query's position become
          // -inf (probability and dS 0), in one block ahead of the
          // probabilities so that those stay free of branches
          if (masked) {
            const int lim = qpos - key0 - 32 * kb - 4 * lgrp;  // keep key offset <= lim
#pragma unroll
            for (int v = 0; v < 16; ++v) sacc[v] = 8 * (v >> 2) + (v & 3) <= lim ? sacc[v] : -INFINITY;
          }
          // dS^T for keys key0 + 32 kb + 8 (v / 4) + 4 lgrp + v % 4
          u32x4 dsf[2];
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              float d2[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int v = 8 * st + 2 * w + u;
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[v], sc, -lse_q));
                d2[u] = p * (dpacc[v] - delta_q);
              }
              dsf[st][w] = pack_f16x2(d2[0], d2[1]);
            }
          // dQ^T += K^T dS^T over the 32 keys of kb
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const unsigned char* kr = sk + (kb * 32 + st * 16) * KROW;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
              dqacc[db] = mfma_f16(tr_read(kr + tro[db][0], kr + tro[db][1]), dsf[st], dqacc[db]);
          }
        }
      }
      wait_loads();
      barrier_nofence();
    };
    int kt = kt_begin;
    for (; kt + 1 < kt_end; kt += 2) {
      step(kt, IC<0>{});
      step(kt + 1, IC<1>{});
    }
    if (kt < kt_end) step(kt, IC<0>{});

    if (!wave_active || !lane_valid) continue;
    const float scl = a.scale;
    float* dst;
    if (!split) {
      dst = a.dq + ((int64_t)b * s.T + t_lane) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH;
    } else {
      const int64_t pidx = (int64_t)(piece_base + slot) * per_bh + bh;
      dst = a.part + (pidx * RBR + (t_lane - g.t0)) * DH;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * lgrp;
        f32x4 v{dqacc[db][4 * j] * scl, dqacc[db][4 * j + 1] * scl, dqacc[db][4 * j + 2] * scl,
                dqacc[db][4 * j + 3] * scl};
        *reinterpret_cast<f32x4*>(dst + d) = v;
      }
  }
}

// Sums the pieces of every split row block, in piece order, into dQ.  One
// thread per (row, 4 head-dim columns); the block is located as in the
// forward's merge (the host's table of split blocks).
template <int DH>
__global__ void attn_bwd_dq_merge_kernel(AttnBwdArgs a) {
  const Shape& s = a.s;
  const int per_bh = s.B * s.Hq;
  constexpr int cols = DH / 4;
  const long long ipb = (long long)per_bh * a.rb * cols;
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
  f32x4 acc{0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < npieces; ++p) {
    const int64_t pidx = (int64_t)(piece_base + p) * per_bh + bh;
    const f32x4 v = *reinterpret_cast<const f32x4*>(a.part + (pidx * a.rb + r) * DH + 4 * c4);
    acc[0] += v[0];
    acc[1] += v[1];
    acc[2] += v[2];
    acc[3] += v[3];
  }
  const int b = bh / s.Hq, qh = bh - b * s.Hq;
  *reinterpret_cast<f32x4*>(a.dq + ((int64_t)b * s.T + t) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH + 4 * c4) = acc;
}

// ---- dK, dV: key-major -----------------------------------------------------
// Work group u: key block kb = u / (B Hkv) (128 keys; lower keys, which more
// of the rank's queries see, come first) of (sequence, kv-head).  It loops
// over the tiles of 64 of the rank's local rows from the first row whose
// position reaches the block's first key (local rows are in increasing
// position order), and over the q-heads of the kv-head's group.  Eight
// waves: wave w takes the 32 keys kg = w % 4 of the block and the 32 rows
// hf = w / 4 of every tile; per (tile, q-head) it computes X = Q K^T and
// dP = dO V^T (its rows x its keys), P and dS, and accumulates
// dV^T += dO^T P and dK^T += Q^T dS over its rows.  The block's K and V rows
// sit in LDS (read once), so a wave holds only its accumulators and two
// waves share a SIMD: one's exp work runs beside the other's products.  At
// the end the two waves of a key group add their sums through LDS (one
// finishes dV, the other dK) and the keys' K/V gradient contributions go to
// the send buffer of the keys' owner ranks (zeros for keys no query of the
// rank sees).
template <int DH>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkv_kernel(AttnBwdArgs a) {
  constexpr int NWV = 8, BQ = 64, KROW = DH * 2, TILE = BQ * KROW;
  constexpr int STAGE = 2 * TILE + 2 * BQ * 4;  // Q | dO | L | Delta
  constexpr int KRPI = 1024 / KROW, TI = BQ / KRPI, QW = 2 * TI / NWV;
  constexpr int NDB = DH / 32, NKS = DH / 16;
  constexpr int KEYS = 128, KV_BYTES = 2 * KEYS * KROW;  // K rows | V rows
  constexpr int KV_INS = KV_BYTES / 1024 / NWV;          // direct loads per wave
  static_assert(QW * NWV == 2 * TI && KV_INS * NWV * 1024 == KV_BYTES, "loads split evenly over the waves");
  // per-lane partial sums of one wave (dV or dK), register-major
  constexpr int PART = NDB * 16 * 64 * 4;
  static_assert(4 * PART <= KV_BYTES && 2 * PART <= STAGE, "the pair sums fit in the freed LDS");
  // the two stages and the K/V rows as three arrays, named at compile time
  // (see stage_mem)
  __shared__ __align__(16) unsigned char smem0[STAGE];
  __shared__ __align__(16) unsigned char smem1[STAGE];
  __shared__ __align__(16) unsigned char kvs[KV_BYTES];
  auto stage_mem = [&](auto ST_) __attribute__((always_inline)) -> unsigned char* {
    if constexpr (decltype(ST_)::value == 0)
      return smem0;
    else
      return smem1;
  };

  const Shape& s = a.s;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int kg = wave & 3, hf = wave >> 2;
  const int per_bg = s.B * s.Hkv;
  const int kb = blockIdx.x / per_bg, bg = blockIdx.x - kb * per_bg;
  const int b = bg / s.Hkv, G = bg - b * s.Hkv;
  const int jsh = G / s.Hkv_s, hk = G - jsh * s.Hkv_s;
  const int grp = s.Hq / s.Hkv;
  const int kvd = s.Hkv_s * DH;
  const int k0 = kb * KEYS, k0w = k0 + 32 * kg;
  const int kpos = k0w + lrow;

  // the block's K and V rows into LDS (rows swizzled as the tiles' rows)
#pragma unroll
  for (int i = 0; i < KV_INS; ++i) {
    const int q = wave + NWV * i;
    const int row = KRPI * q + lane / (KROW / 16);  // 0 .. 2 KEYS - 1: K rows, then V rows
    const int sel = row >= KEYS ? 1 : 0;
    const int r = row - sel * KEYS;
    int key = k0 + r;
    key = key < s.S ? key : s.S - 1;  // keys past the sequence end are never stored
    const uint16_t* src = a.kv + gathered_row(s, jsh, sel, b, key) * kvd + (int64_t)hk * DH;
    attn_load_lds16(src + ((lane % (KROW / 16)) ^ bswz<DH>(r)) * 8, kvs + q * 1024);
  }

  int tro[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    tro[db][0] = tr_offset<DH>(lane, db, 0);
    tro[db][1] = tr_offset<DH>(lane, db, 1);
  }
  const int fl = bswz<DH>(lrow);

  const int t_first = first_row_from(s, k0);
  const int nqt = (s.T + BQ - 1) / BQ;
  const int qt0 = t_first / BQ;
  const int items = t_first < s.T ? (nqt - qt0) * grp : 0;

  // stage of item it: tile qt0 + it / grp, q-head G grp + it % grp
  auto issue = [&](int it, auto ST_) __attribute__((always_inline)) {
    unsigned char* sb = stage_mem(ST_);
    const int t0 = (qt0 + it / grp) * BQ;
    const int qh = G * grp + it % grp;
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int qi = wave + NWV * i;
      const int row = KRPI * (qi % TI) + lane / (KROW / 16);
      int t = t0 + row;
      t = t < s.T ? t : s.T - 1;  // rows past the end are masked
      const uint16_t* src = qi < TI ? a.q + (((int64_t)b * s.Hq + qh) * s.T + t) * DH
                                    : a.dout + ((int64_t)b * s.T + t) * ((int64_t)s.Hq * DH) + (int64_t)qh * DH;
      attn_load_lds16(src + ((lane % (KROW / 16)) ^ bswz<DH>(row)) * 8, sb + qi * 1024);
    }
    if (wave < 2) {
      int t = t0 + lane;
      t = t < s.T ? t : s.T - 1;
      const float* src = (wave == 0 ? a.lse : a.delta) + ((int64_t)b * s.Hq + qh) * s.T + t;
      attn_load_lds4(src, sb + 2 * TILE + wave * BQ * 4);
    }
  };

  f32x16 dvacc[NDB], dkacc[NDB];
#pragma unroll
  for (int x = 0; x < NDB; ++x)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dvacc[x][e] = 0.0f;
      dkacc[x][e] = 0.0f;
    }
  const float sc = a.scale_log2;
  // The lane's key is seen by the local rows [tmin, T): positions grow with
  // the local row, tmin is the first one whose position reaches the key.
  const int tmin = first_row_from(s, kpos);
  const unsigned mspan = (unsigned)(s.T - tmin);
  // the wave's keys' K and V rows (the second operands of X and dP) start
  // at this offset in the K/V array
  const int kvrow = (32 * kg + lrow) * KROW;

  if (items > 0) issue(0, IC<0>{});
  wait_loads();
  barrier_nofence();
  // item it sits in stage it mod 2
  auto step = [&](int it, auto ST_) __attribute__((always_inline)) {
    if (it + 1 < items) issue(it + 1, IC<decltype(ST_)::value ^ 1>{});
    const int t0 = (qt0 + it / grp) * BQ;
    const int th = t0 + 32 * hf;  // the wave's first row
    const int t_last = th + 31 < s.T ? th + 31 : s.T - 1;
    // rows before the wave's first key see none of its keys
    if (th < s.T && local_pos(s, t_last) >= k0w) {
      const bool masked = local_pos(s, th) < k0w + 31 || th + 32 > s.T;
      // re-read the K and V fragments every item instead of keeping them live
      // across the loop (the compiler would hoist the invariant reads and
      // hold 16 more fragments): the offset goes through an empty asm
      int kvo = kvrow;
      asm volatile("" : "+v"(kvo));
      const unsigned char* kw = kvs + kvo;
      const unsigned char* vw = kw + KEYS * KROW;
      const unsigned char* sq = stage_mem(ST_) + 32 * hf * KROW;
      const unsigned char* sd = sq + TILE;
      const float* sl = reinterpret_cast<const float*>(stage_mem(ST_) + 2 * TILE) + 32 * hf;
      const float* sdl = sl + BQ;
      f32x16 xacc, dpacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        xacc[e] = 0.0f;
        dpacc[e] = 0.0f;
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const int off = (((2 * ks + lgrp) ^ fl) << 4);
        const u32x4 kf = *reinterpret_cast<const u32x4*>(kw + off);
        const u32x4 vf = *reinterpret_cast<const u32x4*>(vw + off);
        xacc = mfma_f16(*reinterpret_cast<const u32x4*>(sq + lrow * KROW + off), kf, xacc);
        dpacc = mfma_f16(*reinterpret_cast<const u32x4*>(sd + lrow * KROW + off), vf, dpacc);
      }
      // causal edge and rows past T: scores of rows outside [tmin, T) become
      // -inf (probability and dS 0), in one block ahead of the probabilities
      // so that those stay free of branches
      if (masked) {
        const int mbase = th + 4 * lgrp - tmin;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 8 * (v >> 2) + (v & 3);
          xacc[v] = (unsigned)(mbase + r) < mspan ? xacc[v] : -INFINITY;
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        // registers 8 st .. 8 st + 7 (rows 8 j + 4 lgrp + (0..3) of the
        // wave's 32, j = 2 st, 2 st + 1) form the k-operand of step st
        u32x4 pf, dsf;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const int j = 2 * st + jj;
          const int r0 = 8 * j + 4 * lgrp;
          const f32x4 lv = *reinterpret_cast<const f32x4*>(sl + r0);
          const f32x4 dv = *reinterpret_cast<const f32x4*>(sdl + r0);
          float p[4], d[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int v = 4 * j + u;
            p[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(xacc[v], sc, -lv[u]));
            d[u] = p[u] * (dpacc[v] - dv[u]);
          }
          pf[2 * jj] = pack_f16x2(p[0], p[1]);
          pf[2 * jj + 1] = pack_f16x2(p[2], p[3]);
          dsf[2 * jj] = pack_f16x2(d[0], d[1]);
          dsf[2 * jj + 1] = pack_f16x2(d[2], d[3]);
        }
        const unsigned char* dr = sd + st * 16 * KROW;
        const unsigned char* qr = sq + st * 16 * KROW;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          dvacc[db] = mfma_f16(tr_read(dr + tro[db][0], dr + tro[db][1]), pf, dvacc[db]);
          dkacc[db] = mfma_f16(tr_read(qr + tro[db][0], qr + tro[db][1]), dsf, dkacc[db]);
        }
      }
    }
    wait_loads();
    barrier_nofence();
  };
  int it = 0;
  for (; it + 1 < items; it += 2) {
    step(it, IC<0>{});
    step(it + 1, IC<1>{});
  }
  if (it < items) step(it, IC<0>{});

  // the pair's sums, half the work each: the second-half wave of each key
  // group leaves its dV partial in the K/V rows' array, the first-half wave
  // its dK partial in a stage (every wave is past its last LDS read: the
  // loop ends on a barrier, and with no item the K/V rows were never read);
  // then the first-half wave adds and stores dV, the second-half wave dK
  if (items == 0) {
    wait_loads();  // the K/V rows' loads land before that memory is reused
    barrier_nofence();
  }
  float* pv = reinterpret_cast<float*>(kvs + kg * PART) + lane;
  float* pk = reinterpret_cast<float*>((kg < 2 ? smem0 : smem1) + (kg & 1) * PART) + lane;
  if (hf == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) pv[(db * 16 + e) * 64] = dvacc[db][e];
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) pk[(db * 16 + e) * 64] = dkacc[db][e];
  }
  wait_loads();
  barrier_nofence();
  if (kpos >= s.S) return;
  if (hf == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dvacc[db][e] += pv[(db * 16 + e) * 64];
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) dkacc[db][e] += pk[(db * 16 + e) * 64];
  }
  // owner rank and local row of the key
  int g, t;
  if (s.part == 1) {
    g = kpos % s.D;
    t = kpos / s.D;
  } else {
    const int qc = kpos / s.c;
    g = qc < s.D ? qc : 2 * s.D - 1 - qc;
    t = (qc < s.D ? 0 : s.c) + (kpos - qc * s.c);
  }
  const int64_t kslot = ((((int64_t)g * s.D + jsh) * 2 + 0) * s.B + b) * s.T + t;
  const int64_t vslot = kslot + (int64_t)s.B * s.T;
  float* dk = a.dkv + kslot * kvd + (int64_t)hk * DH;
  float* dv = a.dkv + vslot * kvd + (int64_t)hk * DH;
  const float scl = a.scale;
  if (hf == 0) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * lgrp;
        f32x4 vv4{dvacc[db][4 * j], dvacc[db][4 * j + 1], dvacc[db][4 * j + 2], dvacc[db][4 * j + 3]};
        *reinterpret_cast<f32x4*>(dv + d) = vv4;
      }
  } else {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = db * 32 + 8 * j + 4 * lgrp;
        f32x4 kv4{dkacc[db][4 * j] * scl, dkacc[db][4 * j + 1] * scl, dkacc[db][4 * j + 2] * scl,
                  dkacc[db][4 * j + 3] * scl};
        *reinterpret_cast<f32x4*>(dk + d) = kv4;
      }
  }
}

// ---- host -------------------------------------------------------------------
template <int DH>
static hipError_t launch_bwd_dh(const AttnBwdArgs& a, const AttnPlan& p, hipStream_t st) {
  const Shape& s = a.s;
  const int64_t items = (int64_t)s.M * s.Hq * (DH / 8);
  hipLaunchKernelGGL(attn_bwd_delta_kernel<DH>, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_kernel<DH>, dim3((unsigned)p.units), dim3(256), 0, st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.pieces > 0) {
    const int64_t mitems = (int64_t)p.split_rows * s.B * s.Hq * (DH / 4);
    hipLaunchKernelGGL(attn_bwd_dq_merge_kernel<DH>, dim3((unsigned)((mitems + 255) / 256)), dim3(256), 0, st, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int nkb = (s.S + 127) / 128;
  hipLaunchKernelGGL(attn_bwd_dkv_kernel<DH>, dim3((unsigned)((int64_t)nkb * s.B * s.Hkv)), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd_core(const Shape& s, const uint16_t* q, const uint16_t* kv_gathered, const uint16_t* o,
                                const uint16_t* dout, const float* lse, float* delta, float* dq, float* dkv_send,
                                float* partial, hipStream_t st) {
  // the forward's 4-wave plan (its pieces fit the workspace sized for it)
  const AttnPlan p = attn_plan_shape(s, 4);
  if (p.pieces > 0 && partial == nullptr) return hipErrorInvalidValue;
  AttnBwdArgs a;
  a.q = q;
  a.kv = kv_gathered;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dkv = dkv_send;
  a.part = partial;
  a.s = s;
  a.scale = (float)(1.0 / sqrt((double)s.dh));
  a.scale_log2 = (float)(1.4426950408889634 / sqrt((double)s.dh));
  a.rb = p.rb;
  a.nrb = p.nrb;
  a.kt_max = p.kt_max;
  a.pair = p.pair;
  a.mtab = merge_table(PlanKey{s.c, s.D, s.r, s.part, p.rb, p.nrb, p.kt_max, p.pair});
  if (s.dh == 128) return launch_bwd_dh<128>(a, p, st);
  return launch_bwd_dh<64>(a, p, st);
}

}  // namespace tsp
