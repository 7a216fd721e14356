// Shard GEMMs of the TSP layer on gfx950 matrix cores.
//
// C[m][n] = sum_k A[m][k] * B[n][k]: A holds activations (rows = the rank's
// tokens), B holds nn.Linear-style weights [out][in].  Both are K-contiguous.
// The K axis may be cut into D segments of seg_len (the weight shards of the
// output projection and of the MLP down projection); logical segment s reads
// shard j(s), which is s or, for the MLP ring, (r - s) mod D (Zyphra TSP
// article, "How to Fold a Book": the gated-MLP shards go round a ring and the
// partial outputs are summed locally; the row split of the second matrix sums
// exactly, bowenzhou.top "张量并行", section "机制：行切与列切").
//
// Design: a workgroup of 4 or 8 waves computes a BM x BN tile (x NB weight
// matrices for the fused gate/up product) with 32x32x16 MFMAs, the weight
// tile as the first operand so each lane ends up owning 4 consecutive output
// columns of one row.  Blocks are renumbered so the tiles that share a weight
// block run on the same XCD (blocks are dealt round-robin to the 8 XCDs) and
// hit its L2.  Details of the pipeline are at the kernel below.
#include <stdio.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tsp {

enum { EPI_QKV = 0, EPI_RESID_BF16X = 1, EPI_RESID_F32 = 2, EPI_SWIGLU = 3, EPI_PARTIAL = 4,
       // backward of the gated MLP (see the launchers at the end)
       EPI_SWIGLU_BWD = 5, EPI_DWD = 6, EPI_DWGU = 7,
       // ... with g and u kept from the forward: the dA product's epilogue
       EPI_SWIGLU_KEPT = 8 };

struct GemmArgs {
  const uint16_t* A;
  int64_t lda, a_seg_step;
  const uint16_t* B0;
  const uint16_t* B1;
  int64_t ldb, b_seg_step;
  int32_t M, N, K, seg_len, nseg, ring_rank;
  // epilogue
  float* out;
  uint16_t* out16;
  const void* resid;
  uint16_t* q;
  uint16_t* kv;
  Shape s;
  int32_t src_rank;
  // split-K: nsplit > 1 writes float32 partial sums to partial[split][M][N]
  int32_t nsplit;
  float* partial;
  // backward epilogues: a second float32 output and a second bf16 output;
  // EPI_DWD: columns per weight shard
  float* out2;
  uint16_t* aux16;
  int32_t shard_w;
  // K-major B (the staged kernel's BKM mode): element (k, n) of B, k = kk
  // within K segment j, sits at B0 + j b_seg_step + kk ldbk + col(n) for
  // kk < b_half and at B1 + j b_seg_step + (kk - b_half) ldbk + col(n)
  // otherwise, col(n) = (n / b_w) b_shard + n % b_w (column blocks of b_w,
  // one per weight shard).  N-major B with b_w > 0: row n of B is row
  // (n / b_w) b_shard + n % b_w of the stored matrix (blocks of b_w rows, one
  // per shard, b_shard rows apart); b_w = 0: row n.
  int64_t ldbk, b_shard;
  int32_t b_w, b_half;
  // EPI_SWIGLU_KEPT: u kept from the forward (float32 [M][N]; g is resid)
  const float* resid2;
};

// Stored row of B's row n (N-major B; see GemmArgs::b_w).
__host__ __device__ inline int64_t b_row(const GemmArgs& a, int n) {
  return a.b_w > 0 ? (int64_t)(n / a.b_w) * a.b_shard + n % a.b_w : (int64_t)n;
}

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

// Two floats -> two packed bfloat16, round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// The epilogue inputs of columns n..n+3 of row m, for the epilogues that
// read them (the residual; dA; g and u kept from the forward): loaded apart from the epilogue itself so that a
// tile issues all its input loads before its first store (the stores may
// alias the inputs as far as the compiler knows, so loads placed between
// them would each wait for the previous group's round trip).
// y is read by EPI_SWIGLU_KEPT only (the other epilogues leave it zero and
// the compiler drops it).
struct EpiIn {
  f32x4 x, y;
};

template <int EPI>
__device__ __forceinline__ EpiIn epilogue_input(const GemmArgs& a, int m, int n) {
  EpiIn r{{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  if (m >= a.M || n >= a.N) return r;
  const int64_t off = (int64_t)m * a.N + n;
  if constexpr (EPI == EPI_RESID_BF16X) {
    const u32x2 xr = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.resid) + off);
    r.x[0] = __uint_as_float(xr[0] << 16);
    r.x[1] = __uint_as_float(xr[0] & 0xffff0000u);
    r.x[2] = __uint_as_float(xr[1] << 16);
    r.x[3] = __uint_as_float(xr[1] & 0xffff0000u);
  } else if constexpr (EPI == EPI_RESID_F32 || EPI == EPI_SWIGLU_BWD) {
    if (a.resid != nullptr) r.x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.resid) + off);
  } else if constexpr (EPI == EPI_SWIGLU_KEPT) {
    r.x = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.resid) + off);
    r.y = *reinterpret_cast<const f32x4*>(a.resid2 + off);
  }
  return r;
}

template <int EPI>
constexpr bool epilogue_reads() {
  return EPI == EPI_RESID_BF16X || EPI == EPI_RESID_F32 || EPI == EPI_SWIGLU_BWD || EPI == EPI_SWIGLU_KEPT;
}

// The SwiGLU backward of columns n..n+3 (F axis) of row m from g = x Wg^T,
// u = x Wu^T and dA = dy Wd: with s = sigmoid(g), a = g s u, dU = dA g s,
// dG = dA u s (1 + g (1 - s)).  a goes to out16 (bf16 [M][F]); dG and dU to
// aux16 (bf16 [M][D][2][F/D]: shard j's dG block, then its dU block, per
// row).  The four columns lie in one shard.
__device__ __forceinline__ void swiglu_bwd4(const GemmArgs& a, int m, int n, const float* g4, const float* u4,
                                            const float* da) {
  const Shape& s = a.s;
  const int64_t off = (int64_t)m * a.N + n;
  float av[4], dg[4], du[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float g = g4[e], u = u4[e];
    const float sg = 1.0f / (1.0f + __expf(-g));
    const float gs = g * sg;
    av[e] = gs * u;
    du[e] = da[e] * gs;
    dg[e] = da[e] * u * (sg + gs * (1.0f - sg));
  }
  u32x2 pa{pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
  *reinterpret_cast<u32x2*>(a.out16 + off) = pa;
  const int j = n / s.F_s, f = n - j * s.F_s;
  uint16_t* gu = a.aux16 + (int64_t)m * 2 * s.F + (int64_t)j * 2 * s.F_s + f;
  u32x2 pg{pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3])};
  u32x2 pu{pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3])};
  *reinterpret_cast<u32x2*>(gu) = pg;
  *reinterpret_cast<u32x2*>(gu + s.F_s) = pu;
}

// ein: the epilogue inputs (epilogue_input) for the epilogues that read them.
template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, int m, int n, const float* v,
                                          const float* v2, const EpiIn& ein) {
  if (m >= a.M || n >= a.N) return;
  const f32x4& in = ein.x;
  if constexpr (EPI == EPI_QKV) {
    const Shape& s = a.s;
    const int b = m / s.T, t = m - b * s.T;
    const int j = n / s.nqkv_s;
    int w = n - j * s.nqkv_s;
    uint32_t p0 = pack_f16x2(v[0], v[1]), p1 = pack_f16x2(v[2], v[3]);
    u32x2 pk{p0, p1};
    const int qd = s.Hq_s * s.dh;
    if (w < qd) {
      if (a.q == nullptr) return;
      const int head = j * s.Hq_s + w / s.dh, d = w % s.dh;
      *reinterpret_cast<u32x2*>(a.q + ((((int64_t)b * s.Hq + head) * s.T + t) * s.dh + d)) = pk;
    } else {
      w -= qd;
      const int kvd = s.Hkv_s * s.dh;
      const int sel = w >= kvd ? 1 : 0;
      w -= sel * kvd;
      const int64_t row = ((((int64_t)j * s.D + a.src_rank) * 2 + sel) * s.B + b) * s.T + t;
      *reinterpret_cast<u32x2*>(a.kv + row * kvd + w) = pk;
    }
  } else if constexpr (EPI == EPI_RESID_BF16X) {
    const int64_t off = (int64_t)m * a.N + n;
    f32x4 o;
    o[0] = in[0] + v[0];
    o[1] = in[1] + v[1];
    o[2] = in[2] + v[2];
    o[3] = in[3] + v[3];
    *reinterpret_cast<f32x4*>(a.out + off) = o;
    if (a.out16 != nullptr) {
      u32x2 pk{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(a.out16 + off) = pk;
    }
  } else if constexpr (EPI == EPI_RESID_F32) {
    // float32 residual, or none (the branch alone) when resid is null; the
    // float32 output may be skipped (out null) when only out16 is wanted
    const int64_t off = (int64_t)m * a.N + n;
    f32x4 o{v[0], v[1], v[2], v[3]};
    if (a.resid != nullptr) {
      o[0] = in[0] + v[0];
      o[1] = in[1] + v[1];
      o[2] = in[2] + v[2];
      o[3] = in[3] + v[3];
    }
    if (a.out != nullptr) *reinterpret_cast<f32x4*>(a.out + off) = o;
    if (a.out16 != nullptr) {
      u32x2 pk{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(a.out16 + off) = pk;
    }
  } else if constexpr (EPI == EPI_PARTIAL) {
    // v2 carries the split index in its first element's bits (see caller)
    (void)v2;
  } else if constexpr (EPI == EPI_SWIGLU_BWD) {
    // v = g = x Wg^T, v2 = u = x Wu^T recomputed; in = dA = dy Wd (resid,
    // float32 [M][F])
    const float da[4] = {in[0], in[1], in[2], in[3]};
    swiglu_bwd4(a, m, n, v, v2, da);
  } else if constexpr (EPI == EPI_SWIGLU_KEPT) {
    // v = dA = dy Wd; g and u as the forward wrote them (ein.x, ein.y)
    const float g4[4] = {ein.x[0], ein.x[1], ein.x[2], ein.x[3]};
    const float u4[4] = {ein.y[0], ein.y[1], ein.y[2], ein.y[3]};
    swiglu_bwd4(a, m, n, g4, u4, v);
  } else if constexpr (EPI == EPI_DWD) {
    // C [M][N] (row m = hidden index, column n) -> out [N / w][M][w], w =
    // shard_w: dW_down [D][h][F/D], dW_O [D][h][Hq/D dh]
    const int w = a.shard_w;
    const int j = n / w, f = n - j * w;
    f32x4 o{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(a.out + ((int64_t)j * a.M + m) * w + f) = o;
  } else if constexpr (EPI == EPI_DWGU) {
    // C [2F][h], rows in the [D][2][F/D] order of the dG|dU buffer ->
    // dW_gate (out) or dW_up (out2), both [F][h]
    const Shape& s = a.s;
    const int j = m / (2 * s.F_s);
    const int w = m - j * 2 * s.F_s;
    const bool up = w >= s.F_s;
    const int f = j * s.F_s + (up ? w - s.F_s : w);
    f32x4 o{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>((up ? a.out2 : a.out) + (int64_t)f * a.N + n) = o;
  } else {  // EPI_SWIGLU: v = gate, v2 = up; kept for the backward when out != nullptr
    const int64_t off = (int64_t)m * a.N + n;
    if (a.out != nullptr) {
      *reinterpret_cast<f32x4*>(a.out + off) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(a.out2 + off) = f32x4{v2[0], v2[1], v2[2], v2[3]};
    }
    u32x2 pk{pack_f16x2(silu_f32(v[0]) * v2[0], silu_f32(v[1]) * v2[1]),
             pack_f16x2(silu_f32(v[2]) * v2[2], silu_f32(v[3]) * v2[3])};
    *reinterpret_cast<u32x2*>(a.out16 + off) = pk;
  }
}

__device__ __forceinline__ void seg_offsets(const GemmArgs& a, int k, int64_t& aoff, int64_t& boff) {
  const int sg = k / a.seg_len;
  const int kk = k - sg * a.seg_len;
  int j = sg;
  if (a.ring_rank >= 0) {
    j = a.ring_rank - sg;
    j = j < 0 ? j + a.nseg : j;
  }
  aoff = (int64_t)j * a.a_seg_step + kk;
  boff = (int64_t)j * a.b_seg_step + kk;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void load_lds16(const uint16_t* g, unsigned char* lds) {
  __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_DS_RD = 0x100;

// --------------------------------------------------------------------------
// Kernel: NST-deep LDS ring with every operand copied global -> LDS by direct
// 16-byte loads (global_load_lds_dwordx4: lane i of a wave writes bytes
// [16i, 16i+16) of a 1 KB run), so the loads for tile kt+NST-1 are in flight
// while tile kt is multiplied.  The barrier between K tiles carries no memory
// fence (see lds_barrier).  Weights that must become f16 are converted right
// after their operand read (VALU work that overlaps the other waves' MFMAs).
// LDS rows are BK*2 bytes; 16-byte slot c of row r sits at c ^ swz(r) so the
// 16 rows of one operand read cover the 16 bank groups of the 64-bank LDS.
// Operand reads of the next 16-wide K step are interleaved with this step's
// MFMAs (sched_group_barrier), and the last step's MFMAs run after the
// barrier, overlapping the first operand reads of the next tile.
// Optional split-K (nsplit > 1): unit = (tile, K range), float32 partial tiles
// summed in a fixed order by gemm_reduce_kernel (deterministic).
// --------------------------------------------------------------------------
template <int BK>
__device__ __forceinline__ int gswz(int row) {
  return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// Waits until at most N vector-memory operations of this wave are pending and
// all its LDS operations are done (expcnt untouched).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
}

// Workgroup barrier without the release fence of __syncthreads(): that fence
// makes the compiler wait for every outstanding load, including the tiles
// prefetched for later K steps.  Callers wait for exactly what the next step
// needs (wait_vmcnt) first; the signal fences keep the compiler from moving
// LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Q/K/V scatter of one 32-row x 32-column accumulator block: the column
// block lies inside one head of one shard, so its destination is worked out
// once per block (wave-uniform) and only the row varies per lane.
__device__ __forceinline__ void epi_qkv_block(const GemmArgs& a, int m, int nb0, int lgrp, const f32x16& acc) {
  const Shape& s = a.s;
  if (nb0 >= a.N) return;
  const int j = nb0 / s.nqkv_s;
  int w = nb0 - j * s.nqkv_s;
  const int qd = s.Hq_s * s.dh, kvd = s.Hkv_s * s.dh;
  if (m >= a.M) return;
  const int b = m / s.T, t = m - b * s.T;
  uint16_t* dst;
  if (w < qd) {
    if (a.q == nullptr) return;
    const int head = j * s.Hq_s + w / s.dh, d0 = w % s.dh;
    dst = a.q + ((((int64_t)b * s.Hq + head) * s.T + t) * s.dh + d0);
  } else {
    w -= qd;
    const int sel = w >= kvd ? 1 : 0;
    w -= sel * kvd;
    dst = a.kv + (((((int64_t)j * s.D + a.src_rank) * 2 + sel) * s.B + b) * s.T + t) * kvd + w;
  }
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    u32x2 pk{pack_f16x2(acc[4 * q4], acc[4 * q4 + 1]), pack_f16x2(acc[4 * q4 + 2], acc[4 * q4 + 3])};
    *reinterpret_cast<u32x2*>(dst + 8 * q4 + 4 * lgrp) = pk;
  }
}

// Epilogue of one wave's MB x NBL grid of 32x32 accumulator blocks (x NB
// weight matrices), rows from m_base, columns from n_base.
template <int MB, int NBL, int NB, int EPI>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x16 (&acc)[NB][NBL][MB], int m_base,
                                           int n_base, int lrow, int lgrp, int split) {
#pragma unroll
  for (int y = 0; y < NBL; ++y) {
    // the inputs of this column block's groups first (see epilogue_input),
    // then its stores: MB x 4 loads in flight at a time
    EpiIn in[MB][4];
    if constexpr (epilogue_reads<EPI>()) {
#pragma unroll
      for (int z = 0; z < MB; ++z)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          in[z][q4] = epilogue_input<EPI>(a, m_base + z * 32 + lrow, n_base + y * 32 + 8 * q4 + 4 * lgrp);
    }
#pragma unroll
    for (int z = 0; z < MB; ++z) {
      const int m = m_base + z * 32 + lrow;
      const int nb0 = n_base + y * 32;
      if constexpr (EPI == EPI_QKV) {
        epi_qkv_block(a, m, nb0, lgrp, acc[0][y][z]);
      } else {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int n = nb0 + 8 * q4 + 4 * lgrp;
          float v[4], v2[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            v[e] = acc[0][y][z][4 * q4 + e];
            v2[e] = acc[NB - 1][y][z][4 * q4 + e];
          }
          if constexpr (EPI == EPI_PARTIAL) {
            if (m < a.M && n < a.N) {
              f32x4 o{v[0], v[1], v[2], v[3]};
              *reinterpret_cast<f32x4*>(a.partial + ((int64_t)split * a.M + m) * a.N + n) = o;
            }
          } else if constexpr (epilogue_reads<EPI>()) {
            epilogue4<EPI>(a, m, n, v, v2, in[z][q4]);
          } else {
            epilogue4<EPI>(a, m, n, v, v2, EpiIn{});
          }
        }
      }
    }
  }
}

// Epilogues written as whole rows: each 32 x 32 result block of a wave (both
// weights' blocks for two-weight tiles) goes through the wave's own LDS
// region (row pitch 36 floats: the writes of 16 rows at one column group hit
// 16 distinct bank groups) and is read back as 8 rows x 32 columns per
// instruction, so each store (and epilogue-input load) instruction covers
// whole runs of a row (128 bytes of float32, 64 of a 16-bit output) instead
// of 16 bytes of each of 32 rows: large outputs no longer rely on the L2
// merging partial lines before it evicts them.  LDS operations of one wave
// complete in order, so a wave reads its own writes without a barrier.
constexpr int kRowPitch = 36;
template <int NB>
constexpr int rows_lds_floats() {
  return NB * 32 * kRowPitch;
}
template <int MB, int NBL, int NB, int EPI>
__device__ __forceinline__ void store_tile_rows(const GemmArgs& a, const f32x16 (&acc)[NB][NBL][MB], int m_base,
                                                int n_base, int lane, float* lds, int split) {
  constexpr int P = kRowPitch;
  const int lrow = lane & 31, lgrp = lane >> 5;
  const int rr = lane >> 3, cc = (lane & 7) * 4;
#pragma unroll
  for (int y = 0; y < NBL; ++y)
#pragma unroll
    for (int z = 0; z < MB; ++z) {
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 v{acc[x][y][z][4 * q4], acc[x][y][z][4 * q4 + 1], acc[x][y][z][4 * q4 + 2],
                        acc[x][y][z][4 * q4 + 3]};
          *reinterpret_cast<f32x4*>(lds + (x * 32 + lrow) * P + 8 * q4 + 4 * lgrp) = v;
        }
      EpiIn in[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (epilogue_reads<EPI>())
          in[i] = epilogue_input<EPI>(a, m_base + z * 32 + rr + 8 * i, n_base + y * 32 + cc);
        else
          in[i] = EpiIn{};
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m_base + z * 32 + rr + 8 * i, n = n_base + y * 32 + cc;
        const f32x4 v = *reinterpret_cast<const f32x4*>(lds + (rr + 8 * i) * P + cc);
        const f32x4 w = *reinterpret_cast<const f32x4*>(lds + ((NB - 1) * 32 + rr + 8 * i) * P + cc);
        const float vv[4] = {v[0], v[1], v[2], v[3]};
        const float ww[4] = {w[0], w[1], w[2], w[3]};
        if constexpr (EPI == EPI_PARTIAL) {
          if (m < a.M && n < a.N)
            *reinterpret_cast<f32x4*>(a.partial + ((int64_t)split * a.M + m) * a.N + n) = v;
        } else {
          epilogue4<EPI>(a, m, n, vv, ww, in[i]);
        }
      }
    }
}

template <int BM, int BN, int NB, int WGM, int NW, int BK, int NST, bool SEGFAST, bool F16, bool CONVB, int EPI,
          int OCC>
__global__ __launch_bounds__(64 * NW, OCC) void gemm_kernel(GemmArgs a) {
  constexpr int WGN = NW / WGM;
  constexpr int ROWB = BK * 2, SLOTS = BK / 8, RPI = 1024 / ROWB;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int MB = WM / 32, NBL = WN / 32;
  constexpr int BROWS = NB * BN;
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + BROWS) * ROWB;
  constexpr int QA = BM / RPI;                   // direct-load instructions of the A tile
  constexpr int QT = (BM + BROWS) / RPI;         // ... of the whole stage
  constexpr int QI = (QT + NW - 1) / NW;         // per wave, at most
  constexpr int C_HI = QI, C_LO = QT / NW;       // per-wave counts (waves < QT % NW have C_HI)
  constexpr int KS = BK / 16;
  constexpr int NFRAG = MB + NB * NBL;
  constexpr int NMFMA = MB * NB * NBL;
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(NST >= 2 && NST <= 5, "stages");
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(BM % RPI == 0 && BROWS % RPI == 0, "load split");
  static_assert((NST - 2) * C_HI < 64, "vmcnt range");
  __shared__ __align__(16) unsigned char smem[NST * STAGE];

  // wave index made scalar so everything derived from it (load roles, LDS
  // offsets, segment selects) stays in SGPRs
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;
  const bool hi_count = (QT % NW == 0) || (wave < QT % NW);

  const int mtiles = (a.M + BM - 1) / BM;
  const int ntiles = mtiles * ((a.N + BN - 1) / BN);
  const int units = ntiles * a.nsplit;
  int u;
  {
    const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    const int q = units >> 3, rem = units & 7;
    u = xcd * q + (xcd < rem ? xcd : rem) + idx;
  }
  // tiles in groups of 8 row tiles, row tile fastest inside a group: the
  // tiles an XCD runs at once share 8 A row blocks and a few B column blocks
  // in its L2 (the weight-gradient products' operands are far larger than
  // one L2)
  const int tile = u % ntiles, split = u / ntiles;
  constexpr int GM = 8;
  const int ntn = (a.N + BN - 1) / BN;
  const int group = tile / (GM * ntn), first_m = group * GM;
  const int gsz = mtiles - first_m < GM ? mtiles - first_m : GM;
  const int gin = tile - group * (GM * ntn);
  const int mt = first_m + gin % gsz, nt = gin / gsz;
  const int m0 = mt * BM, n0 = nt * BN;
  const int nk_all = a.K / BK;
  const int per = (nk_all + a.nsplit - 1) / a.nsplit;
  const int kt0 = split * per;
  const int kt1 = (kt0 + per < nk_all) ? kt0 + per : nk_all;

  // direct loads: instruction q writes LDS rows RPI q ..; lane i lands in row
  // RPI q + i / SLOTS at physical slot i % SLOTS (logical slot ^ swizzle)
  // When NW divides both instruction counts, whether load i is an A or a B
  // load and whether it exists at all are compile-time facts.
  constexpr bool STATIC_ROLES = (QA % NW == 0) && (QT % NW == 0);
  const uint16_t* src[QI];
  int chunk[QI];
  bool isb[QI];
#pragma unroll
  for (int i = 0; i < QI; ++i) {
    const int q = wave + NW * i;
    const int row = RPI * q + lane / SLOTS;
    chunk[i] = (lane % SLOTS) ^ gswz<BK>(row);
    isb[i] = STATIC_ROLES ? (NW * i >= QA) : (q >= QA);
    if (!isb[i]) {
      int m = m0 + row;
      m = m < a.M ? m : a.M - 1;
      src[i] = a.A + (int64_t)m * a.lda;
    } else {
      const int brow = row - BM;
      const int which = brow / BN;
      int n = n0 + brow - which * BN;
      n = n < a.N ? n : a.N - 1;
      src[i] = ((NB == 2 && which == 1) ? a.B1 : a.B0) + b_row(a, n) * a.ldb;
    }
    if constexpr (SEGFAST) src[i] += chunk[i] * 8;
  }
  // K cursor of the next tile to load (segment s, offset kk inside it)
  int cur_s = 0, cur_kk = 0;
  if constexpr (SEGFAST) {
    const int k = kt0 * BK;
    cur_s = k / a.seg_len;
    cur_kk = k - cur_s * a.seg_len;
  }
  auto issue_loads = [&](int kt, int stage) {
    unsigned char* sbase = smem + stage * STAGE;
    int64_t aoff_u = 0, boff_u = 0;
    if constexpr (SEGFAST) {
      int j = cur_s;
      if (a.ring_rank >= 0) {
        j = a.ring_rank - cur_s;
        j = j < 0 ? j + a.nseg : j;
      }
      aoff_u = (int64_t)j * a.a_seg_step + cur_kk;
      boff_u = (int64_t)j * a.b_seg_step + cur_kk;
      cur_kk += BK;
      if (cur_kk >= a.seg_len) {
        cur_kk -= a.seg_len;
        ++cur_s;
      }
    }
#pragma unroll
    for (int i = 0; i < QI; ++i) {
      const int q = wave + NW * i;
      if (STATIC_ROLES || q < QT) {
        int64_t off;
        if constexpr (SEGFAST) {
          off = isb[i] ? boff_u : aoff_u;
        } else {
          int64_t ao, bo;
          seg_offsets(a, kt * BK + chunk[i] * 8, ao, bo);
          off = isb[i] ? bo : ao;
        }
        load_lds16(src[i] + off, sbase + q * 1024);
      }
    }
  };

  f32x16 acc[NB][NBL][MB];
#pragma unroll
  for (int x = 0; x < NB; ++x)
#pragma unroll
    for (int y = 0; y < NBL; ++y)
#pragma unroll
      for (int z = 0; z < MB; ++z)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[x][y][z][e] = 0.0f;

  const int lrow = lane & 31, lgrp = lane >> 5, lsw = gswz<BK>(lane & 31);
  u32x4 af[2][MB], bf[2][NB][NBL];
  auto read_frags = [&](int stage, int ks, int buf) {
    const unsigned char* sa = smem + stage * STAGE;
    const unsigned char* sb = sa + A_BYTES;
    const int pch = ((2 * ks + lgrp) ^ lsw) << 4;
#pragma unroll
    for (int z = 0; z < MB; ++z)
      af[buf][z] = *reinterpret_cast<const u32x4*>(sa + (wm * WM + z * 32 + lrow) * ROWB + pch);
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int y = 0; y < NBL; ++y)
        bf[buf][x][y] = *reinterpret_cast<const u32x4*>(sb + (x * BN + wn * WN + y * 32 + lrow) * ROWB + pch);
  };
  auto mfmas = [&](int buf) {
    if constexpr (CONVB) {
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int y = 0; y < NBL; ++y) bf[buf][x][y] = bf16x8_to_f16x8(bf[buf][x][y]);
    }
#pragma unroll
    for (int x = 0; x < NB; ++x)
#pragma unroll
      for (int y = 0; y < NBL; ++y)
#pragma unroll
        for (int z = 0; z < MB; ++z) {
          if constexpr (F16)
            acc[x][y][z] = mfma_f16(bf[buf][x][y], af[buf][z], acc[x][y][z]);
          else
            acc[x][y][z] = mfma_bf16(bf[buf][x][y], af[buf][z], acc[x][y][z]);
        }
  };
  auto schedule_step = [&]() {
    constexpr int NPAIR = NFRAG < NMFMA ? NFRAG : NMFMA;
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
    }
    if constexpr (NMFMA > NPAIR) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NMFMA - NPAIR, 0);
    if constexpr (NFRAG > NPAIR) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, NFRAG - NPAIR, 0);
  };
  // Waits until this wave's loads of all but the newest `newer` issued tiles
  // have landed (loads complete in issue order) and its LDS reads are done.
  // The LDS wait is a separate instruction on every path so the compiler
  // knows no LDS read is pending after it, whatever branch the vmcnt wait took.
  auto wait_tile = [&](int newer) {
    wait_vmcnt<63>();
    if constexpr (NST >= 5) {
      if (newer >= 3) {
        if (hi_count) wait_vmcnt<3 * C_HI>(); else wait_vmcnt<3 * C_LO>();
        return;
      }
    }
    if constexpr (NST >= 4) {
      if (newer >= 2) {
        if (hi_count) wait_vmcnt<2 * C_HI>(); else wait_vmcnt<2 * C_LO>();
        return;
      }
    }
    if constexpr (NST >= 3) {
      if (newer >= 1) {
        if (hi_count) wait_vmcnt<C_HI>(); else wait_vmcnt<C_LO>();
        return;
      }
    }
    wait_vmcnt<0>();
  };
  // Steady-state wait: the newest NST - 2 tiles may stay in flight.
  auto wait_steady = [&]() {
    if constexpr (QT % NW == 0) {
      wait_vmcnt<(NST - 2) * C_HI>();
    } else {
      wait_vmcnt<63>();
      if (hi_count) wait_vmcnt<(NST - 2) * C_HI>(); else wait_vmcnt<(NST - 2) * C_LO>();
    }
  };
  // The rest of a K tile after its first 16-wide step: the remaining steps
  // (operand reads of step ks + 1 overlapping the MFMAs of step ks), the wait
  // for the next tile, the barrier, and the last step's MFMAs overlapping the
  // next tile's first operand reads (which, on the last tile, read a stage
  // that is never used: kept unconditional so the reads and the MFMAs share a
  // basic block and the compiler does not wait for the reads).
  int stage = 0;
  auto finish_tile = [&](bool steady) {
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
      read_frags(stage, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
      schedule_step();
    }
    // keep every MFMA of the step above the wait and the barrier
    __builtin_amdgcn_sched_barrier(0);
    if (steady) wait_steady(); else wait_vmcnt<0>();
    lds_barrier();
    const int nstage = stage + 1 == NST ? 0 : stage + 1;
    read_frags(nstage, 0, 0);
    mfmas((KS - 1) & 1);
    schedule_step();
    stage = nstage;
  };

  if (kt0 < kt1) {
    int issued = 0;
#pragma unroll
    for (int i = 0; i < NST - 1; ++i)
      if (kt0 + i < kt1) {
        issue_loads(kt0 + i, i);
        ++issued;
      }
    wait_tile(issued - 1);
    lds_barrier();
    read_frags(0, 0, 0);
  }
  int kt = kt0;
  // steady state: every iteration issues the tile NST - 1 ahead
  for (; kt + NST - 1 < kt1; ++kt) {
    int fill = stage + NST - 1;
    fill = fill >= NST ? fill - NST : fill;
    issue_loads(kt + NST - 1, fill);
    finish_tile(true);
  }
  // drain: nothing left to issue
  for (; kt < kt1; ++kt) finish_tile(false);

  if constexpr (EPI != EPI_QKV) {
    static_assert(NW * rows_lds_floats<NB>() * 4 <= NST * STAGE, "row staging fits the operand stages");
    __syncthreads();  // every wave is done with the operand stages
    store_tile_rows<MB, NBL, NB, EPI>(a, acc, m0 + wm * WM, n0 + wn * WN, lane,
                                      reinterpret_cast<float*>(smem) + wave * rows_lds_floats<NB>(), split);
  } else {
    store_tile<MB, NBL, NB, EPI>(a, acc, m0 + wm * WM, n0 + wn * WN, lrow, lgrp, split);
  }
}

// --------------------------------------------------------------------------
// Register-staged kernel (NW waves, accumulators in AGPRs).  K steps of 64
// so that each row of a tile is one whole 128-byte line, read by 8 lanes with
// 16-byte loads.  Global loads run PF K tiles ahead into PF register sets; a
// landed tile is written into the free one of two LDS stages (the weights
// converted bf16 -> f16 on the way when CONVB, once per tile rather than once
// per operand read).  Thread t stages the 16-byte slot t % 8 of rows
// t / 8 + (NW * 8) i of the tile, so all its loads share one K offset.
// Offsets are 32-bit byte offsets from a wave-uniform base (the launcher
// checks the operands fit in 4 GiB).
// --------------------------------------------------------------------------
constexpr int SG_DS_WR = 0x200, SG_VMEM_RD = 0x020;

// Schedule of the K step that also stages a tile: MFMA i is followed by one
// operand read of the next step and by an even share of the tile's LDS
// writes (and of the loads that refill the freed registers).
template <int I, int NMFMA, int NFRAG, int CPT, bool LOADS>
__device__ __forceinline__ void sched_stage_one() {
  constexpr int PER = (CPT + NMFMA - 1) / NMFMA;
  constexpr int done = I * PER;
  constexpr int w = done >= CPT ? 0 : (CPT - done < PER ? CPT - done : PER);
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
  if constexpr (I < NFRAG) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
  if constexpr (w > 0) {
    __builtin_amdgcn_sched_group_barrier(SG_DS_WR, w, 0);
    if constexpr (LOADS) __builtin_amdgcn_sched_group_barrier(SG_VMEM_RD, w, 0);
  }
  if constexpr (I == NMFMA - 1 && NFRAG > NMFMA) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, NFRAG - NMFMA, 0);
}
template <int NMFMA, int NFRAG, int CPT, bool LOADS, int... I>
__device__ __forceinline__ void sched_stage_step(std::integer_sequence<int, I...>) {
  (sched_stage_one<I, NMFMA, NFRAG, CPT, LOADS>(), ...);
}

// Transposing LDS read of two 4-row groups (rows r and r + 4 of one column
// per lane): the 8 k-values of a K-major operand fragment.
typedef short gv4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) gv4i16 lds_gv4i16;
__device__ __forceinline__ u32x4 tr_read2(const unsigned char* p0, const unsigned char* p1) {
  const gv4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_gv4i16*)p0);
  const gv4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_gv4i16*)p1);
  const u32x2 h0 = __builtin_bit_cast(u32x2, r0), h1 = __builtin_bit_cast(u32x2, r1);
  return u32x4{h0[0], h0[1], h1[0], h1[1]};
}

// BKM: B is K-major (a weight read as stored, for the backward products).
// Its stage holds the tile's 64 k-rows of BN columns (2 BN bytes each) as
// 16-byte runs of 8 columns, swizzled so that the transposing reads of 4
// consecutive k-rows (32 bytes of each) hit 4 different 64-byte bank windows;
// a fragment (8 consecutive k of one column) is two transposing reads.
// Physical run of logical run `run` of k-row k: inside each whole group of 16
// runs, run XOR 4 (k % 4); in the 8-run tail of a 192-column row (384 bytes,
// so consecutive rows start half a bank cycle apart), run XOR 4 ((k / 2) % 2).
template <int RUNS>
__device__ __forceinline__ int bkm_run(int run, int k) {
  constexpr int FULL = RUNS & ~15;
  static_assert(RUNS == FULL || RUNS - FULL == 8, "whole 16-run groups and at most an 8-run tail");
  return run < FULL ? run ^ ((k & 3) << 2) : FULL + ((run - FULL) ^ (((k >> 1) & 1) << 2));
}
template <int BM, int BN, int NB, int WGM, int NW, bool SEGFAST, bool F16, bool CONVB, int EPI, int NSTG,
          bool SPLIT, bool BKM = false>
__global__ __launch_bounds__(64 * NW, 1) void gemm_staged_kernel(GemmArgs a) {
  // LDS rows of 64 K-values padded from 128 to 144 bytes: the 16 rows one
  // operand read touches then start in 16 different bank groups, and the
  // K step and stage enter the read address as immediates
  constexpr int BK = 64, ROWB = 144;
  // SPLIT (two weights): the wave columns take one weight each over the
  // whole BN columns (wave column 0 W_0, column 1 W_1) instead of both
  // weights over BN / WGN columns, so a wave reads half the weight rows per
  // MFMA; the epilogue pairs the two results through LDS.
  constexpr int WGN = NW / WGM;
  static_assert(!SPLIT || (NB == 2 && WGN == 2), "split needs two weights and two wave columns");
  constexpr int NBW = SPLIT ? 1 : NB;   // weights per wave
  constexpr int WM = BM / WGM, WN = SPLIT ? BN : BN / WGN;
  constexpr int MB = WM / 32, NBL = WN / 32;
  static_assert(!SPLIT || MB % 2 == 0, "split pairs halves of the wave rows");
  static_assert(!BKM || (NB == 1 && !SPLIT && !CONVB && SEGFAST && (BN == 128 || BN == 192 || BN == 256) &&
                         EPI != EPI_QKV),
                "K-major B mode");
  constexpr int R = BM + NB * BN;       // LDS rows per stage (N-major B)
  constexpr int STAGE = BKM ? BM * ROWB + BK * 2 * BN : R * ROWB;
  constexpr int RS = 8 * NW;            // rows covered by one chunk round
  constexpr int CPT = R / RS;           // staged 16-byte chunks per thread per tile
  constexpr int CA = BM / RS;           // ... of which rows of A
  constexpr int KS = BK / 16;
  constexpr int RUNS = BN / 8;          // BKM: 16-byte runs per k-row
  constexpr int NFRAG = MB + (BKM ? 2 : 1) * NBW * NBL, NMFMA = MB * NBW * NBL;
  static_assert(NW % WGM == 0 && WM % 32 == 0 && WN % 32 == 0, "wave tile");
  static_assert(BM % RS == 0, "chunk rounds must not straddle A and B");
  static_assert(NB == 2 || BN % RS == 0, "a single weight fills whole chunk rounds");
  static_assert(2 * STAGE <= 160 * 1024, "LDS");
  __shared__ __align__(16) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave % WGM, wn = wave / WGM;

  const int mtiles = (a.M + BM - 1) / BM;
  const int ntiles = mtiles * ((a.N + BN - 1) / BN);
  const int units = ntiles * a.nsplit;
  int u;
  {
    const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    const int q = units >> 3, rem = units & 7;
    u = xcd * q + (xcd < rem ? xcd : rem) + idx;
  }
  const int tile = u % ntiles, split = u / ntiles;
  const int mt = tile % mtiles, nt_ = tile / mtiles;
  const int m0 = mt * BM, n0 = nt_ * BN;
  const int nk_all = a.K / BK;
  const int per = (nk_all + a.nsplit - 1) / a.nsplit;
  const int kt0 = split * per;
  const int kt1 = (kt0 + per < nk_all) ? kt0 + per : nk_all;
  const int ntile = kt1 > kt0 ? kt1 - kt0 : 0;

  // staging roles
  const int crow = tid >> 3, cslot = tid & 7;
  // byte offset of the chunk's row (+ its slot when the K cursor is uniform;
  // a per-lane cursor already includes the slot), K offset excluded
  const int slot_k = SEGFAST ? cslot * 8 : 0;
  uint32_t goff[CPT];
  // BKM: each B chunk's k-row in the tile, column offset col(n) and LDS offset
  int bkrow[BKM ? CPT - CA : 1], blds[BKM ? CPT - CA : 1];
  int64_t bcol[BKM ? CPT - CA : 1];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int row = crow + RS * i;
    if constexpr (BKM) {
      if (i >= CA) {
        const int c = (i - CA) * (64 * NW) + tid;
        const int krow = c / RUNS, run = c % RUNS;
        int n = n0 + run * 8;
        n = n < a.N ? n : a.N - 8;  // N is a multiple of 8
        bkrow[i - CA] = krow;
        bcol[i - CA] = (int64_t)(n / a.b_w) * a.b_shard + n % a.b_w;
        blds[i - CA] = BM * ROWB + krow * (2 * BN) + (bkm_run<RUNS>(run, krow) << 4);
        goff[i] = 0;
        continue;
      }
    }
    if (i < CA) {
      int m = m0 + row;
      m = m < a.M ? m : a.M - 1;
      goff[i] = (uint32_t)(((int64_t)m * a.lda + slot_k) * 2);
    } else {
      // B rows [0, BN) are W_0's, [BN, 2 BN) W_1's; a round of RS rows may
      // straddle the two when BN is not a multiple of RS
      const int brow = row - BM;
      const int which = brow >= BN ? 1 : 0;
      int n = n0 + brow - which * BN;
      n = n < a.N ? n : a.N - 1;
      goff[i] = (uint32_t)((b_row(a, n) * a.ldb + slot_k) * 2);
    }
  }
  const uint32_t lds_w = crow * ROWB + cslot * 16;

  // K cursor of the next tile to load: uniform when segments are whole
  // multiples of 64, else per lane (its slot may cross a segment boundary
  // at a different tile than other slots).  Loads past the last tile reload
  // the last one (kept in ak/bk), so every iteration has the same shape.
  int cur_s, cur_kk, nload = 0;
  {
    const int k = kt0 * BK + (SEGFAST ? 0 : cslot * 8);
    cur_s = k / a.seg_len;
    cur_kk = k - cur_s * a.seg_len;
  }
  uint32_t ak = 0, bk = 0;
  int tj = 0, tkk = 0;  // BKM: segment and offset in it of the last tile loaded
  // NSTG register sets of staged chunks: loads run NSTG tiles ahead of the
  // LDS stage they are written to
  static_assert(NSTG == 1 || NSTG == 2, "one or two register sets");
  u32x4 stg[NSTG][CPT];
  // offsets of the next tile to load (advances the K cursor)
  auto next_offsets = [&]() __attribute__((always_inline)) {
    if (nload < ntile) {
      int j = cur_s;
      if (a.ring_rank >= 0) {
        j = a.ring_rank - cur_s;
        j = j < 0 ? j + a.nseg : j;
      }
      ak = (uint32_t)(((int64_t)j * a.a_seg_step + cur_kk) * 2);
      bk = (uint32_t)(((int64_t)j * a.b_seg_step + cur_kk) * 2);
      tj = j;
      tkk = cur_kk;
      cur_kk += BK;
      if (cur_kk >= a.seg_len) {
        cur_kk -= a.seg_len;
        ++cur_s;
      }
    }
    ++nload;
  };
  auto load_chunk = [&](u32x4& dst, int i) __attribute__((always_inline)) {
    const unsigned char* base;
    uint32_t off = goff[i];
    if (i < CA) {
      base = reinterpret_cast<const unsigned char*>(a.A);
      off += ak;
    } else if constexpr (BKM) {
      const int kk = tkk + bkrow[i - CA];
      const bool hi = kk >= a.b_half;
      base = reinterpret_cast<const unsigned char*>(hi ? a.B1 : a.B0);
      off = (uint32_t)(((int64_t)tj * a.b_seg_step + (int64_t)(hi ? kk - a.b_half : kk) * a.ldbk + bcol[i - CA]) * 2);
    } else {
      const int first = (RS * i - BM) / BN, last = (RS * i + RS - 1 - BM) / BN;  // compile-time
      int which = first;
      if (first != last) which = (crow + RS * i - BM) >= BN ? 1 : 0;            // straddling round
      base = reinterpret_cast<const unsigned char*>((NB == 2 && which == 1) ? a.B1 : a.B0);
      off += bk;
    }
    dst = *reinterpret_cast<const u32x4*>(base + off);
  };
  auto write_chunk = [&](const u32x4& src, int i, int stage) __attribute__((always_inline)) {
    u32x4 v = src;
    if constexpr (CONVB) {
      if (i >= CA) v = bf16x8_to_f16x8(v);
    }
    const int lo = (BKM && i >= CA) ? blds[BKM ? i - CA : 0] : lds_w + i * RS * ROWB;
    *reinterpret_cast<u32x4*>(smem + stage * STAGE + lo) = v;
  };
  auto load_tile = [&](u32x4 (&dst)[CPT]) __attribute__((always_inline)) {
    next_offsets();
#pragma unroll
    for (int i = 0; i < CPT; ++i) load_chunk(dst[i], i);
  };

  f32x16 acc[NBW][NBL][MB];
#pragma unroll
  for (int x = 0; x < NBW; ++x)
#pragma unroll
    for (int y = 0; y < NBL; ++y)
#pragma unroll
      for (int z = 0; z < MB; ++z)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[x][y][z][e] = 0.0f;

  const int lrow = lane & 31, lgrp = lane >> 5;
  // BKM: byte offsets (within a 16-row K step of the B stage) of the two
  // transposing reads of column block y: lane (gq = lane / 16, sl = lane %
  // 16) points at row 8 (gq / 2) + sl / 4 (+ 4) and columns wn WN + 32 y +
  // 16 (gq % 2) + 4 (sl % 4) .. + 3, and receives column wn WN + 32 y +
  // lane % 32, rows 8 (lane / 32) + (0..7)
  int btr[BKM ? NBL : 1][2];
  if constexpr (BKM) {
    const int gq = lane >> 4, sl = lane & 15;
#pragma unroll
    for (int y = 0; y < NBL; ++y)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 8 * (gq >> 1) + (sl >> 2) + 4 * h;
        const int c = wn * WN + 32 * y + 16 * (gq & 1) + 4 * (sl & 3);
        btr[y][h] = r * (2 * BN) + (bkm_run<RUNS>(c >> 3, r) << 4) + (c & 7) * 2;
      }
  }
  u32x4 af[2][MB], bf[2][NBW][NBL];
  auto read_frags = [&](int stage, int ks, int buf) __attribute__((always_inline)) {
    const unsigned char* sa = smem + stage * STAGE;
    const unsigned char* sb = sa + BM * ROWB;
    const int pch = (2 * ks + lgrp) << 4;
#pragma unroll
    for (int z = 0; z < MB; ++z)
      af[buf][z] = *reinterpret_cast<const u32x4*>(sa + (wm * WM + z * 32 + lrow) * ROWB + pch);
    if constexpr (BKM) {
      const unsigned char* sk = sb + ks * 16 * (2 * BN);
#pragma unroll
      for (int y = 0; y < NBL; ++y) bf[buf][0][y] = tr_read2(sk + btr[y][0], sk + btr[y][1]);
    } else {
#pragma unroll
      for (int x = 0; x < NBW; ++x)
#pragma unroll
        for (int y = 0; y < NBL; ++y) {
          const int brow = SPLIT ? wn * BN + y * 32 : x * BN + wn * WN + y * 32;
          bf[buf][x][y] = *reinterpret_cast<const u32x4*>(sb + (brow + lrow) * ROWB + pch);
        }
    }
  };
  auto mfmas = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < NBW; ++x)
#pragma unroll
      for (int y = 0; y < NBL; ++y)
#pragma unroll
        for (int z = 0; z < MB; ++z) {
          if constexpr (F16)
            acc[x][y][z] = mfma_f16(bf[buf][x][y], af[buf][z], acc[x][y][z]);
          else
            acc[x][y][z] = mfma_bf16(bf[buf][x][y], af[buf][z], acc[x][y][z]);
        }
  };
  // one MFMA, then one operand read of the next step, and so on
  auto schedule_step = [&]() __attribute__((always_inline)) {
    constexpr int NPAIR = NFRAG < NMFMA ? NFRAG : NMFMA;
#pragma unroll
    for (int i = 0; i < NPAIR; ++i) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_RD, 1, 0);
    }
    if constexpr (NMFMA > NPAIR) __builtin_amdgcn_sched_group_barrier(SG_MFMA, NMFMA - NPAIR, 0);
    if constexpr (NFRAG > NPAIR) __builtin_amdgcn_sched_group_barrier(SG_DS_RD, NFRAG - NPAIR, 0);
  };
  // LDS wait + workgroup barrier (no memory fence: see lds_barrier)
  auto sync = [&]() __attribute__((always_inline)) {
    wait_vmcnt<63>();
    lds_barrier();
  };

  // One K tile in LDS stage P.  MODE 0: also write register set 1 - P (the
  // next tile) into the other stage, chunk by chunk over the K steps, and
  // refill each chunk's registers with the tile two further on; MODE 1:
  // last tile.
  constexpr int CH = (CPT + KS - 2) / (KS - 1);  // chunks staged per K step
  auto iteration = [&](auto P_, auto MODE_) __attribute__((always_inline)) {
    constexpr int P = decltype(P_)::value, MODE = decltype(MODE_)::value;
    if constexpr (MODE == 0) next_offsets();
    static_for<0, KS - 1>([&](auto KS_) __attribute__((always_inline)) {
      constexpr int ks = decltype(KS_)::value;
      read_frags(P, ks + 1, (ks + 1) & 1);
      mfmas(ks & 1);
      if constexpr (MODE == 0) {
        constexpr int NC = CPT - ks * CH < CH ? CPT - ks * CH : CH;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          write_chunk(stg[NSTG == 2 ? 1 - P : 0][ks * CH + c], ks * CH + c, 1 - P);
          load_chunk(stg[NSTG == 2 ? 1 - P : 0][ks * CH + c], ks * CH + c);
        }
        sched_stage_step<NMFMA, NFRAG, NC, true>(std::make_integer_sequence<int, NMFMA>{});
      } else {
        schedule_step();
      }
    });
    if constexpr (MODE == 0) {
      __builtin_amdgcn_sched_barrier(0);
      sync();
      read_frags(1 - P, 0, 0);
    }
    mfmas((KS - 1) & 1);
    if constexpr (MODE == 0) schedule_step();
  };

  if (ntile > 0) {
    load_tile(stg[0]);
    if constexpr (NSTG == 2) load_tile(stg[NSTG - 1]);
#pragma unroll
    for (int i = 0; i < CPT; ++i) write_chunk(stg[0][i], i, 0);
    load_tile(stg[0]);
    sync();
    read_frags(0, 0, 0);
    int t = 0;
    for (; t + 1 < ntile; t += 2) {
      iteration(IC<0>{}, IC<0>{});
      iteration(IC<1>{}, IC<0>{});
    }
    if (t < ntile) iteration(IC<0>{}, IC<1>{});
  }
  if constexpr (SPLIT) {
    // Waves (wm, 0) and (wm, 1) hold W_0 and W_1 results for the same WM x BN
    // block, in the same lane layout.  Wave column 0 finishes the first half
    // of the row blocks, column 1 the second: each writes the half it does
    // not finish to LDS (register-major, lane-minor: conflict-free), and
    // reads its partner's matching half.
    constexpr int HB = MB / 2;                        // row blocks per half
    constexpr int XF = NBL * HB * 16;                 // floats exchanged per lane
    static_assert(NW * 64 * XF * 4 <= 2 * STAGE, "exchange fits in the stages");
    float* xch = reinterpret_cast<float*>(smem);
    wait_vmcnt<63>();                                 // (waits for this wave's LDS operations)
    lds_barrier();                                    // every wave's last operand reads are done
    // (register indices stay compile-time: the wave column only selects)
    const bool col0 = wn == 0;
    {
      float* mine = xch + (wave * XF) * 64 + lane;
#pragma unroll
      for (int y = 0; y < NBL; ++y)
#pragma unroll
        for (int z = 0; z < HB; ++z)
#pragma unroll
          for (int e = 0; e < 16; ++e)  // the half the partner finishes
            mine[((y * HB + z) * 16 + e) * 64] = col0 ? acc[0][y][z + HB][e] : acc[0][y][z][e];
    }
    wait_vmcnt<63>();
    lds_barrier();
    f32x16 pair[2][NBL][HB];                          // [W_0, W_1][col block][row block of the half]
    {
      const int partner = wm + WGM * (1 - wn);
      const float* theirs = xch + (partner * XF) * 64 + lane;
#pragma unroll
      for (int y = 0; y < NBL; ++y)
#pragma unroll
        for (int z = 0; z < HB; ++z)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float t = theirs[((y * HB + z) * 16 + e) * 64];
            const float own = col0 ? acc[0][y][z][e] : acc[0][y][z + HB][e];  // the half this wave finishes
            pair[0][y][z][e] = col0 ? own : t;
            pair[1][y][z][e] = col0 ? t : own;
          }
    }
    static_assert(NW * rows_lds_floats<2>() * 4 <= 2 * STAGE, "row staging fits in the stages");
    wait_vmcnt<63>();
    lds_barrier();                                    // every wave has read its partner's half
    store_tile_rows<HB, NBL, 2, EPI>(a, pair, m0 + wm * WM + (wn == 0 ? 0 : HB * 32), n0, lane,
                                     reinterpret_cast<float*>(smem) + wave * rows_lds_floats<2>(), split);
  } else if constexpr (EPI != EPI_QKV) {
    static_assert(NW * rows_lds_floats<NB>() * 4 <= 2 * STAGE, "row staging fits in the stages");
    wait_vmcnt<63>();
    lds_barrier();                                    // every wave's last operand reads are done
    store_tile_rows<MB, NBL, NB, EPI>(a, acc, m0 + wm * WM, n0 + wn * WN, lane,
                                      reinterpret_cast<float*>(smem) + wave * rows_lds_floats<NB>(), split);
  } else {
    store_tile<MB, NBL, NB, EPI>(a, acc, m0 + wm * WM, n0 + wn * WN, lrow, lgrp, split);
  }
}

// Sums the split-K partials in split order and applies the residual epilogue:
// out = resid + sum_p partial[p]  (resid bf16 when EPI == EPI_RESID_BF16X,
// float32 when EPI_RESID_F32), plus the f16 copy when out16 != nullptr.
// A thread takes four consecutive columns of RR rows at a time (rows
// RR y, RR y + 1, ... then RR (y + gridDim.y), ...) and issues every load of
// those rows before its first store (the stores may alias the partials as far
// as the compiler knows, so it would not move later rows' loads above them).
constexpr int kReduceRows = 4;
template <int EPI>
__global__ void gemm_reduce_kernel(GemmArgs a) {
  constexpr int RR = kReduceRows;
  const int n = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (n >= a.N) return;
  const int64_t plane = (int64_t)a.M * a.N;
  for (int m0 = blockIdx.y * RR; m0 < a.M; m0 += gridDim.y * RR) {
    f32x4 acc[RR];
    EpiIn in[RR];
    int64_t off[RR];
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      const int m = m0 + i < a.M ? m0 + i : a.M - 1;  // rows past M: loaded, not stored
      off[i] = (int64_t)m * a.N + n;
      acc[i] = *reinterpret_cast<const f32x4*>(a.partial + off[i]);
      in[i] = epilogue_input<EPI>(a, m0 + i, n);
    }
    for (int p = 1; p < a.nsplit; ++p) {
      f32x4 t[RR];
#pragma unroll
      for (int i = 0; i < RR; ++i) t[i] = *reinterpret_cast<const f32x4*>(a.partial + p * plane + off[i]);
#pragma unroll
      for (int i = 0; i < RR; ++i) {
        acc[i][0] += t[i][0];
        acc[i][1] += t[i][1];
        acc[i][2] += t[i][2];
        acc[i][3] += t[i][3];
      }
    }
#pragma unroll
    for (int i = 0; i < RR; ++i) {
      float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
      epilogue4<EPI>(a, m0 + i, n, v, v, in[i]);
    }
  }
}

static dim3 reduce_grid(const GemmArgs& a) {
  const int rows = (a.M + kReduceRows - 1) / kReduceRows;
  return dim3((unsigned)((a.N / 4 + 255) / 256), (unsigned)(rows < 65535 ? rows : 65535));
}

// --------------------------------------------------------------------------
// Host-side tile choice and launch
// --------------------------------------------------------------------------
template <int BM, int BN, int NB, int WGM, int NW, int BK, int NST, bool SEGFAST, bool F16, bool CONVB, int EPI,
          int OCC>
static hipError_t launch_tile_seg(GemmArgs a, int nsplit, hipStream_t st) {
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  if constexpr (EPI == EPI_RESID_F32 || EPI == EPI_RESID_BF16X) {
    if (nsplit > 1 && a.partial != nullptr) {
      a.nsplit = nsplit;
      hipLaunchKernelGGL((gemm_kernel<BM, BN, NB, WGM, NW, BK, NST, SEGFAST, F16, CONVB, EPI_PARTIAL, OCC>),
                         dim3(mt * nt * nsplit), dim3(64 * NW), 0, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_reduce_kernel<EPI>),
                         reduce_grid(a), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  a.nsplit = 1;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, NB, WGM, NW, BK, NST, SEGFAST, F16, CONVB, EPI, OCC>), dim3(mt * nt),
                     dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

// Segments that are whole multiples of BK never split a K tile, so the
// segment cursor can be kept per tile instead of per lane.
template <int BM, int BN, int NB, int WGM, int NW, int BK, int NST, bool F16, bool CONVB, int EPI, int OCC>
static hipError_t launch_tile(GemmArgs a, int nsplit, hipStream_t st) {
  if (a.seg_len % BK == 0)
    return launch_tile_seg<BM, BN, NB, WGM, NW, BK, NST, true, F16, CONVB, EPI, OCC>(a, nsplit, st);
  return launch_tile_seg<BM, BN, NB, WGM, NW, BK, NST, false, F16, CONVB, EPI, OCC>(a, nsplit, st);
}

// The staged kernel addresses its operands with 32-bit byte offsets.
static bool staged_fits(const GemmArgs& a) {
  const int64_t seg_extra = a.seg_len;
  const int64_t a_end = ((int64_t)(a.M - 1) * a.lda + (int64_t)(a.nseg - 1) * a.a_seg_step + seg_extra) * 2;
  const int64_t b_end = (b_row(a, a.N - 1) * a.ldb + (int64_t)(a.nseg - 1) * a.b_seg_step + seg_extra) * 2;
  return a_end < ((int64_t)1 << 32) - 64 && b_end < ((int64_t)1 << 32) - 64 && a.K % 64 == 0;
}

template <int BM, int BN, int NB, int WGM, int NW, bool SEGFAST, bool F16, bool CONVB, int EPI, int NSTG, bool SPLIT,
          bool BKM = false>
static hipError_t launch_staged_seg(GemmArgs a, int nsplit, hipStream_t st) {
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  if constexpr (EPI == EPI_RESID_F32 || EPI == EPI_RESID_BF16X) {
    if (nsplit > 1 && a.partial != nullptr) {
      a.nsplit = nsplit;
      hipLaunchKernelGGL((gemm_staged_kernel<BM, BN, NB, WGM, NW, SEGFAST, F16, CONVB, EPI_PARTIAL, NSTG, SPLIT, BKM>),
                         dim3(mt * nt * nsplit), dim3(64 * NW), 0, st, a);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      hipLaunchKernelGGL((gemm_reduce_kernel<EPI>),
                         reduce_grid(a), dim3(256), 0, st, a);
      return hipGetLastError();
    }
  }
  a.nsplit = 1;
  hipLaunchKernelGGL((gemm_staged_kernel<BM, BN, NB, WGM, NW, SEGFAST, F16, CONVB, EPI, NSTG, SPLIT, BKM>), dim3(mt * nt),
                     dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

// Returns hipErrorNotSupported (nothing launched) when the operands are too
// large for 32-bit offsets; callers then use the direct-load kernel.
template <int BM, int BN, int NB, int WGM, int NW, bool F16, bool CONVB, int EPI, int NSTG = 1, bool SPLIT = false>
static hipError_t launch_staged(const GemmArgs& a, int nsplit, hipStream_t st) {
  if (!staged_fits(a)) return hipErrorNotSupported;
  if (a.seg_len % 64 == 0)
    return launch_staged_seg<BM, BN, NB, WGM, NW, true, F16, CONVB, EPI, NSTG, SPLIT>(a, nsplit, st);
  return launch_staged_seg<BM, BN, NB, WGM, NW, false, F16, CONVB, EPI, NSTG, SPLIT>(a, nsplit, st);
}

// K-major B (BKM): bf16 operands, segments whole multiples of 64, N and the
// column blocks multiples of 8, every operand within 32-bit byte offsets of
// its base.  hipErrorInvalidValue (nothing launched) otherwise.
static bool bkm_fits(const GemmArgs& a) {
  if (a.K % 64 != 0 || a.seg_len % 64 != 0 || a.N % 8 != 0 || a.b_w % 8 != 0 || a.b_half <= 0 ||
      a.b_half > a.seg_len)
    return false;
  const int64_t lim = ((int64_t)1 << 32) - 64;
  const int64_t a_end = ((int64_t)(a.M - 1) * a.lda + (int64_t)(a.nseg - 1) * a.a_seg_step + a.seg_len) * 2;
  const int64_t col_end = (int64_t)((a.N - 1) / a.b_w) * a.b_shard + a.b_w;
  const int64_t rows = a.b_half > a.seg_len - a.b_half ? a.b_half : a.seg_len - a.b_half;
  const int64_t b_end = ((int64_t)(a.nseg - 1) * a.b_seg_step + (rows - 1) * a.ldbk + col_end) * 2;
  return a_end < lim && b_end < lim;
}

template <int BM, int BN, int WGM, int NW, int EPI>
static hipError_t launch_staged_bkm(const GemmArgs& a, int nsplit, hipStream_t st) {
  if (!bkm_fits(a)) return hipErrorInvalidValue;
  return launch_staged_seg<BM, BN, 1, WGM, NW, true, false, false, EPI, 1, false, true>(a, nsplit, st);
}

// Overrides set through tsp_set_tuning (for tests and tuning): a GEMM
// configuration index and, for the output and down projections, a split-K
// factor.  -1: the default dispatch.
enum { KNOB_GEMM_QKV = 0, KNOB_GEMM_OPROJ = 1, KNOB_GEMM_GATEUP = 2, KNOB_GEMM_DOWN = 3,
       KNOB_SPLIT_OPROJ = 4, KNOB_SPLIT_DOWN = 5 };

// Single-weight GEMM configurations:
//   0: staged, 256x192 tile, 8 waves (4x2)   -- Q/K/V projection; output and
//      down projections without split-K when it takes fewer rounds
//   1: staged, 256x128 tile, 4 waves (2x2)
//   2: staged, 256x192 tile, 4 waves (2x2)
//   3: direct-load ring, 256x256 tile, 8 waves, K step 32, 5 stages
//   4: staged, 128x128 tile, 4 waves (2x2);  5: staged, 128x128 tile, 8 waves (2x4)
//   6: staged, 256x128 tile, 8 waves (4x2)   -- output and down projections
//   7: as 6 with loads two tiles ahead of their LDS write (two register sets)
// The staged configurations otherwise keep one register set (loads one tile
// ahead): measured as fast or faster, with 8 x CPT fewer VGPRs.
// The staged kernel needs 32-bit operand offsets; beyond that the direct-load
// ring kernel (64-bit addressing) runs instead.
template <bool F16, bool CONVB, int EPI>
static hipError_t launch_cfg(const GemmArgs& a, int cfg, int nsplit, hipStream_t st) {
  hipError_t e = hipErrorNotSupported;
  switch (cfg) {
    case 0: e = launch_staged<256, 192, 1, 4, 8, F16, CONVB, EPI>(a, nsplit, st); break;
    case 1: e = launch_staged<256, 128, 1, 2, 4, F16, CONVB, EPI>(a, nsplit, st); break;
    case 2: e = launch_staged<256, 192, 1, 2, 4, F16, CONVB, EPI>(a, nsplit, st); break;
    case 4: e = launch_staged<128, 128, 1, 2, 4, F16, CONVB, EPI>(a, nsplit, st); break;
    case 5: e = launch_staged<128, 128, 1, 2, 8, F16, CONVB, EPI>(a, nsplit, st); break;
    case 6: e = launch_staged<256, 128, 1, 4, 8, F16, CONVB, EPI>(a, nsplit, st); break;
    case 7: e = launch_staged<256, 128, 1, 4, 8, F16, CONVB, EPI, 2>(a, nsplit, st); break;
    default: break;
  }
  if (e != hipErrorNotSupported) return e;
  return launch_tile<256, 256, 1, 2, 8, 32, 5, F16, CONVB, EPI, 1>(a, nsplit, st);
}

template <bool F16, bool CONVB, int EPI>
static hipError_t launch_single(const GemmArgs& a, int knob_cfg, int knob_split, int max_split, hipStream_t st) {
  // Q/K/V: 256x192 tiles; output/down (M x h): 256x128 tiles, split along K
  // as planned by gemm_split_plan so that tiles x splits covers the CUs
  int cfg = EPI == EPI_QKV ? 0 : 6, nsplit = EPI == EPI_QKV ? 1 : max_split;
  const int over_cfg = tune_get(knob_cfg);
  if (over_cfg >= 0) cfg = over_cfg;
  if (knob_split >= 0 && tune_get(knob_split) >= 1) nsplit = tune_get(knob_split);
  // the workspace holds partials for at most the planned factor
  if (nsplit < 1 || nsplit > max_split || a.partial == nullptr) nsplit = 1;
  if (EPI != EPI_QKV && over_cfg < 0 && nsplit == 1) {
    // Unsplit output/down projection (large M): 256x192 tiles when their
    // work-group rounds on 256 CUs, at 1.3x the time of a 256x128 tile (1.5x
    // the products, fewer LDS operand reads per product), finish sooner.
    const long long mt = (a.M + 255) / 256;
    const long long r192 = (mt * ((a.N + 191) / 192) + 255) / 256;
    const long long r128 = (mt * ((a.N + 127) / 128) + 255) / 256;
    if (13 * r192 < 10 * r128) cfg = 0;
  }
  return launch_cfg<F16, CONVB, EPI>(a, cfg, nsplit, st);
}

static GemmArgs base_args(const Shape& s) {
  GemmArgs a{};
  a.s = s;
  a.ring_rank = -1;
  a.nseg = 1;
  a.nsplit = 1;
  return a;
}

hipError_t launch_qkv_gemm(const Shape& s, int src_rank, const uint16_t* x, const uint16_t* w_qkv,
                           uint16_t* q, uint16_t* kv_gathered, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = x;
  a.lda = s.h;
  a.B0 = a.B1 = w_qkv;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.D * s.nqkv_s;
  a.K = s.h;
  a.seg_len = s.h;
  a.q = q;
  a.kv = kv_gathered;
  a.src_rank = src_rank;
  return launch_single<false, false, EPI_QKV>(a, KNOB_GEMM_QKV, -1, 1, st);
}

hipError_t launch_oproj_gemm(const Shape& s, const uint16_t* o, const uint16_t* w_o,
                             const uint16_t* x_resid, const float* resid_f32, float* out, uint16_t* out16,
                             float* partial, hipStream_t st) {
  GemmArgs a = base_args(s);
  const int seg = s.Hq_s * s.dh;
  a.A = o;
  a.lda = (int64_t)s.Hq * s.dh;
  a.a_seg_step = seg;
  a.B0 = a.B1 = w_o;
  a.ldb = seg;
  a.b_seg_step = (int64_t)s.h * seg;
  a.M = s.M;
  a.N = s.h;
  a.K = s.Hq * s.dh;
  a.seg_len = seg;
  a.nseg = s.D;
  a.out = out;
  a.out16 = out16;
  a.partial = partial;
  if (x_resid != nullptr) {
    a.resid = x_resid;
    return launch_single<true, true, EPI_RESID_BF16X>(a, KNOB_GEMM_OPROJ, KNOB_SPLIT_OPROJ, gemm_split_plan(s), st);
  }
  a.resid = resid_f32;
  return launch_single<true, true, EPI_RESID_F32>(a, KNOB_GEMM_OPROJ, KNOB_SPLIT_OPROJ, gemm_split_plan(s), st);
}

hipError_t launch_gateup_gemm(const Shape& s, const uint16_t* x, bool x_bf16, const uint16_t* w_g,
                              const uint16_t* w_u, uint16_t* act, hipStream_t st, float* gu_keep) {
  GemmArgs a = base_args(s);
  if (gu_keep != nullptr) {
    a.out = gu_keep;
    a.out2 = gu_keep + (int64_t)s.M * s.F;
  }
  a.A = x;
  a.lda = s.h;
  a.B0 = w_g;
  a.B1 = w_u;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.F;
  a.K = s.h;
  a.seg_len = s.h;
  a.out16 = act;
  // Dual-weight (gate and up) configurations:
  //   0: staged, 128x192 (x2) tile, 8 waves (4x2);  1: staged, 128x192 (x2), 4 waves (2x2)
  //   2: direct-load ring, 128x128 (x2), 4 waves, K step 64, 3 stages
  //   3: staged, 256x96 (x2) tile, 8 waves (8x1);  4: as 3 with two register sets
  //   5: staged, 256x96 (x2) tile, 8 waves (4x2) with one weight per wave column
  // bf16 input: both operands bf16 as given (bf16 matrix cores), the
  // default tile only
  if (x_bf16) {
    hipError_t e = launch_staged<256, 96, 2, 4, 8, false, false, EPI_SWIGLU, 1, true>(a, 1, st);
    if (e != hipErrorNotSupported) return e;
    return launch_tile<128, 128, 2, 2, 4, 64, 3, false, false, EPI_SWIGLU, 1>(a, 1, st);
  }
  int cfg = tune_get(KNOB_GEMM_GATEUP);
  if (cfg < 0) cfg = 5;
  hipError_t e = hipErrorNotSupported;
  if (cfg == 0) e = launch_staged<128, 192, 2, 4, 8, true, true, EPI_SWIGLU>(a, 1, st);
  if (cfg == 1) e = launch_staged<128, 192, 2, 2, 4, true, true, EPI_SWIGLU>(a, 1, st);
  if (cfg == 3) e = launch_staged<256, 96, 2, 8, 8, true, true, EPI_SWIGLU>(a, 1, st);
  if (cfg == 4) e = launch_staged<256, 96, 2, 8, 8, true, true, EPI_SWIGLU, 2>(a, 1, st);
  if (cfg == 5) e = launch_staged<256, 96, 2, 4, 8, true, true, EPI_SWIGLU, 1, true>(a, 1, st);
  if (e != hipErrorNotSupported) return e;
  return launch_tile<128, 128, 2, 2, 4, 64, 3, true, true, EPI_SWIGLU, 1>(a, 1, st);
}

hipError_t launch_down_gemm(const Shape& s, const uint16_t* act, const uint16_t* w_d,
                            const float* resid, float* y, float* partial, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = act;
  a.lda = s.F;
  a.a_seg_step = s.F_s;
  a.B0 = a.B1 = w_d;
  a.ldb = s.F_s;
  a.b_seg_step = (int64_t)s.h * s.F_s;
  a.M = s.M;
  a.N = s.h;
  a.K = s.F;
  a.seg_len = s.F_s;
  a.nseg = s.D;
  a.ring_rank = s.r;
  a.out = y;
  a.resid = resid;
  a.partial = partial;
  return launch_single<true, true, EPI_RESID_F32>(a, KNOB_GEMM_DOWN, KNOB_SPLIT_DOWN, gemm_split_plan(s), st);
}

// --------------------------------------------------------------------------
// Backward of the gated MLP (bf16 matrix cores on bf16 operands; gradients
// keep bf16's float32 range).  Operand layouts (NT form, K-contiguous):
//   dA   = dy16 [M][h] x WdT [F][h]                  -> float32 dA [M][F]
//   g, u = x [M][h] x (Wg, Wu) [F][h], epilogue       -> a [M][F], dG|dU
//   dx   = dGU [M][D][2][F/D] x WguT [h][D][2][F/D]   (K segments per shard,
//          in ring order (r - s) mod D)  + dx_resid  -> float32 dx [M][h]
//   dWd  = dyT [h][Mp] x aT [F][Mp]                   -> dW_down [D][h][F/D]
//   dWgu = dGUT [2F][Mp] x xT [h][Mp]                 -> dW_gate, dW_up [F][h]
// Mp = M rounded up to 64 (the transposed copies are zero beyond M).
// --------------------------------------------------------------------------
hipError_t launch_bwd_da(const Shape& s, const uint16_t* dy16, const uint16_t* wdT, float* da, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dy16;
  a.lda = s.h;
  a.B0 = a.B1 = wdT;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.F;
  a.K = s.h;
  a.seg_len = s.h;
  a.out = da;
  a.resid = nullptr;
  return launch_cfg<false, false, EPI_RESID_F32>(a, 0, 1, st);
}

hipError_t launch_bwd_da_kept(const Shape& s, const uint16_t* dy16, const uint16_t* wdT, const float* gu_keep,
                              uint16_t* act16, uint16_t* dgu, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dy16;
  a.lda = s.h;
  a.B0 = a.B1 = wdT;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.F;
  a.K = s.h;
  a.seg_len = s.h;
  a.resid = gu_keep;
  a.resid2 = gu_keep + (int64_t)s.M * s.F;
  a.out16 = act16;
  a.aux16 = dgu;
  return launch_cfg<false, false, EPI_SWIGLU_KEPT>(a, 0, 1, st);
}

hipError_t launch_bwd_gu(const Shape& s, const uint16_t* x, bool x_bf16, const uint16_t* w_g, const uint16_t* w_u,
                         const float* da, uint16_t* act16, uint16_t* dgu, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = x;
  a.lda = s.h;
  a.B0 = w_g;
  a.B1 = w_u;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.F;
  a.K = s.h;
  a.seg_len = s.h;
  a.resid = da;
  a.out16 = act16;
  a.aux16 = dgu;
  hipError_t e;
  if (x_bf16) {
    e = launch_staged<256, 96, 2, 4, 8, false, false, EPI_SWIGLU_BWD, 1, true>(a, 1, st);
    if (e != hipErrorNotSupported) return e;
    return launch_tile<128, 128, 2, 2, 4, 64, 3, false, false, EPI_SWIGLU_BWD, 1>(a, 1, st);
  }
  e = launch_staged<256, 96, 2, 4, 8, true, true, EPI_SWIGLU_BWD, 1, true>(a, 1, st);
  if (e != hipErrorNotSupported) return e;
  return launch_tile<128, 128, 2, 2, 4, 64, 3, true, true, EPI_SWIGLU_BWD, 1>(a, 1, st);
}

hipError_t launch_bwd_dx(const Shape& s, const uint16_t* dgu, const uint16_t* wguT, const float* dx_resid, float* dx,
                         float* partial, hipStream_t st) {
  GemmArgs a = base_args(s);
  const int seg = 2 * s.F_s;
  a.A = dgu;
  a.lda = 2 * (int64_t)s.F;
  a.a_seg_step = seg;
  a.B0 = a.B1 = wguT;
  a.ldb = 2 * (int64_t)s.F;
  a.b_seg_step = seg;
  a.M = s.M;
  a.N = s.h;
  a.K = 2 * s.F;
  a.seg_len = seg;
  a.nseg = s.D;
  a.ring_rank = s.r;
  a.out = dx;
  a.resid = dx_resid;
  a.partial = partial;
  return launch_single<false, false, EPI_RESID_F32>(a, -1, -1, gemm_split_plan(s), st);
}

hipError_t launch_bwd_dwd(const Shape& s, int m_pad, const uint16_t* dyT, const uint16_t* aT, float* dw_down,
                          hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dyT;
  a.lda = m_pad;
  a.B0 = a.B1 = aT;
  a.ldb = m_pad;
  a.M = s.h;
  a.N = s.F;
  a.K = m_pad;
  a.seg_len = m_pad;
  a.out = dw_down;
  a.shard_w = s.F_s;
  return launch_cfg<false, false, EPI_DWD>(a, 3, 1, st);  // 256x256: short contraction over the tokens
}

hipError_t launch_bwd_dwgu(const Shape& s, int m_pad, const uint16_t* dguT, const uint16_t* xT, float* dw_gate,
                           float* dw_up, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dguT;
  a.lda = m_pad;
  a.B0 = a.B1 = xT;
  a.ldb = m_pad;
  a.M = 2 * s.F;
  a.N = s.h;
  a.K = m_pad;
  a.seg_len = m_pad;
  a.out = dw_gate;
  a.out2 = dw_up;
  return launch_cfg<false, false, EPI_DWGU>(a, 3, 1, st);  // 256x256: short contraction over the tokens
}

// ---- backward of the attention (projections) --------------------------------
// q = x Wq^T for the rank's tokens, Wq [Hq*dh][h] the Q rows of every shard:
// the Q/K/V epilogue with every column a Q column (a shard of Hq/D dh).
hipError_t launch_q_gemm(const Shape& s, const uint16_t* x, const uint16_t* w_qkv, uint16_t* q, hipStream_t st) {
  Shape sq = s;
  sq.nqkv_s = s.Hq_s * s.dh;
  GemmArgs a = base_args(sq);
  a.A = x;
  a.lda = s.h;
  // the Q rows of every shard of W_QKV: Hq/D dh rows at the start of each
  // shard's nqkv_s rows
  a.B0 = a.B1 = w_qkv;
  a.ldb = s.h;
  a.b_w = s.Hq_s * s.dh;
  a.b_shard = s.nqkv_s;
  a.M = s.M;
  a.N = s.Hq * s.dh;
  a.K = s.h;
  a.seg_len = s.h;
  a.q = q;
  a.kv = nullptr;
  a.src_rank = s.r;
  // 128x128 tiles: N = Hq dh alone gives few 256-row tiles (88 at the 8K layer)
  return launch_cfg<false, false, EPI_QKV>(a, 5, 1, st);
}

// dO = dh16 WoT^T stored f16 [M][Hq*dh]; WoT [Hq*dh][h] bf16.
hipError_t launch_attn_bwd_do(const Shape& s, const uint16_t* dh16, const uint16_t* woT, uint16_t* dout,
                              hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dh16;
  a.lda = s.h;
  a.B0 = a.B1 = woT;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.Hq * s.dh;
  a.K = s.h;
  a.seg_len = s.h;
  a.out = nullptr;
  a.out16 = dout;
  a.resid = nullptr;
  return launch_cfg<false, false, EPI_RESID_F32>(a, 5, 1, st);  // as launch_q_gemm
}

// dW_O [D][h][Hq/D dh] = dhT oT^T (both [.][m_pad] bf16).
hipError_t launch_attn_bwd_dwo(const Shape& s, int m_pad, const uint16_t* dhT, const uint16_t* oT, float* dw_o,
                               hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = dhT;
  a.lda = m_pad;
  a.B0 = a.B1 = oT;
  a.ldb = m_pad;
  a.M = s.h;
  a.N = s.Hq * s.dh;
  a.K = m_pad;
  a.seg_len = m_pad;
  a.out = dw_o;
  a.shard_w = s.Hq_s * s.dh;
  return launch_cfg<false, false, EPI_DWD>(a, 3, 1, st);  // 256x256: short contraction over the tokens
}

// dx = dx_resid + sum over the shards (ring order) of G_j WqkvT_j^T, G [M][D
// nqkv_s] the packed dQ | dK | dV rows of every shard, WqkvT [h][D nqkv_s].
hipError_t launch_attn_bwd_dx(const Shape& s, const uint16_t* g16, const uint16_t* wqkvT, const float* dx_resid,
                              float* dx, float* partial, hipStream_t st) {
  GemmArgs a = base_args(s);
  const int seg = s.nqkv_s;
  a.A = g16;
  a.lda = (int64_t)s.D * seg;
  a.a_seg_step = seg;
  a.B0 = a.B1 = wqkvT;
  a.ldb = (int64_t)s.D * seg;
  a.b_seg_step = seg;
  a.M = s.M;
  a.N = s.h;
  a.K = s.D * seg;
  a.seg_len = seg;
  a.nseg = s.D;
  a.ring_rank = s.r;
  a.out = dx;
  a.resid = dx_resid;
  a.partial = partial;
  return launch_single<false, false, EPI_RESID_F32>(a, -1, -1, gemm_split_plan(s), st);
}

// dW_QKV [D nqkv_s][h] = gT xT^T (both [.][m_pad] bf16): the packed layout.
hipError_t launch_attn_bwd_dwqkv(const Shape& s, int m_pad, const uint16_t* gT, const uint16_t* xT, float* dw_qkv,
                                 hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = gT;
  a.lda = m_pad;
  a.B0 = a.B1 = xT;
  a.ldb = m_pad;
  a.M = s.D * s.nqkv_s;
  a.N = s.h;
  a.K = m_pad;
  a.seg_len = m_pad;
  a.out = dw_qkv;
  a.resid = nullptr;
  // short contraction (the tokens): 256x256 tiles, fewer operand bytes per product
  return launch_cfg<false, false, EPI_RESID_F32>(a, 3, 1, st);
}

// --------------------------------------------------------------------------
// Backward products with the weight read as stored (K-major B: the staged
// kernel's BKM mode), no transposed copy:
//   KMAJ_DA      dA  = dy16 W_down      W_down [D][h][F/D]: K = h, a column
//                                       block of F/D per shard
//   KMAJ_DX_MLP  dx  = dx_resid + sum over the shards (ring order) of
//                      dG_j W_gate,j + dU_j W_up,j   (K segment j = the
//                      2 F/D columns [dG_j | dU_j] of dGU; its first F/D
//                      rows from W_gate [F][h], the rest from W_up)
//   KMAJ_DO      dO  = dh16 W_O         W_O [D][h][Hq/D dh]: K = h
//   KMAJ_DX_ATTN dx  = dx_resid + G W_QKV  W_QKV [D nqkv_s][h], K segments
//                      of nqkv_s in ring order
// --------------------------------------------------------------------------
static GemmArgs kmajor_args(const Shape& s, int use) {
  GemmArgs a = base_args(s);
  a.M = s.M;
  switch (use) {
    case KMAJ_DA:
      a.lda = s.h;
      a.N = s.F;
      a.K = a.seg_len = a.b_half = s.h;
      a.ldbk = a.b_w = s.F_s;
      a.b_shard = (int64_t)s.h * s.F_s;
      break;
    case KMAJ_DX_MLP:
      a.lda = 2 * (int64_t)s.F;
      a.a_seg_step = 2 * s.F_s;
      a.N = s.h;
      a.K = 2 * s.F;
      a.seg_len = 2 * s.F_s;
      a.b_half = s.F_s;
      a.nseg = s.D;
      a.ring_rank = s.r;
      a.ldbk = a.b_w = s.h;
      a.b_seg_step = (int64_t)s.F_s * s.h;
      break;
    case KMAJ_DO:
      a.lda = s.h;
      a.N = s.Hq * s.dh;
      a.K = a.seg_len = a.b_half = s.h;
      a.ldbk = a.b_w = s.Hq_s * s.dh;
      a.b_shard = (int64_t)s.h * s.Hq_s * s.dh;
      break;
    default:  // KMAJ_DX_ATTN
      a.lda = (int64_t)s.D * s.nqkv_s;
      a.a_seg_step = s.nqkv_s;
      a.N = s.h;
      a.K = s.D * s.nqkv_s;
      a.seg_len = a.b_half = s.nqkv_s;
      a.nseg = s.D;
      a.ring_rank = s.r;
      a.ldbk = a.b_w = s.h;
      a.b_seg_step = (int64_t)s.nqkv_s * s.h;
      break;
  }
  return a;
}

bool kmajor_ok(const Shape& s, int use) { return bkm_fits(kmajor_args(s, use)); }

hipError_t launch_bwd_da_kmajor(const Shape& s, const uint16_t* dy16, const uint16_t* w_down, float* da,
                                hipStream_t st) {
  GemmArgs a = kmajor_args(s, KMAJ_DA);
  a.A = dy16;
  a.B0 = a.B1 = w_down;
  a.out = da;
  a.resid = nullptr;
  // 256x192 tiles: one round of work groups at the 8K layer (4 x 58 tiles)
  return launch_staged_bkm<256, 192, 4, 8, EPI_RESID_F32>(a, 1, st);
}

hipError_t launch_bwd_da_kept_kmajor(const Shape& s, const uint16_t* dy16, const uint16_t* w_down,
                                     const float* gu_keep, uint16_t* act16, uint16_t* dgu, hipStream_t st) {
  GemmArgs a = kmajor_args(s, KMAJ_DA);
  a.A = dy16;
  a.B0 = a.B1 = w_down;
  a.resid = gu_keep;
  a.resid2 = gu_keep + (int64_t)s.M * s.F;
  a.out16 = act16;
  a.aux16 = dgu;
  return launch_staged_bkm<256, 192, 4, 8, EPI_SWIGLU_KEPT>(a, 1, st);
}

hipError_t launch_bwd_dx_kmajor(const Shape& s, const uint16_t* dgu, const uint16_t* w_g, const uint16_t* w_u,
                                const float* dx_resid, float* dx, float* partial, hipStream_t st) {
  GemmArgs a = kmajor_args(s, KMAJ_DX_MLP);
  a.A = dgu;
  a.B0 = w_g;
  a.B1 = w_u;
  a.out = dx;
  a.resid = dx_resid;
  a.partial = partial;
  return launch_staged_bkm<256, 128, 4, 8, EPI_RESID_F32>(a, partial != nullptr ? gemm_split_plan(s) : 1, st);
}

hipError_t launch_attn_bwd_do_kmajor(const Shape& s, const uint16_t* dh16, const uint16_t* w_o, uint16_t* dout,
                                     hipStream_t st) {
  GemmArgs a = kmajor_args(s, KMAJ_DO);
  a.A = dh16;
  a.B0 = a.B1 = w_o;
  a.out = nullptr;
  a.out16 = dout;
  a.resid = nullptr;
  return launch_staged_bkm<128, 128, 2, 8, EPI_RESID_F32>(a, 1, st);
}

hipError_t launch_attn_bwd_dx_kmajor(const Shape& s, const uint16_t* g16, const uint16_t* w_qkv,
                                     const float* dx_resid, float* dx, float* partial, hipStream_t st) {
  GemmArgs a = kmajor_args(s, KMAJ_DX_ATTN);
  a.A = g16;
  a.B0 = a.B1 = w_qkv;
  a.out = dx;
  a.resid = dx_resid;
  a.partial = partial;
  return launch_staged_bkm<256, 128, 4, 8, EPI_RESID_F32>(a, partial != nullptr ? gemm_split_plan(s) : 1, st);
}

__global__ void f32_to_f16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n4) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n4; i += stride) {
    f32x4 v = reinterpret_cast<const f32x4*>(x)[i];
    u32x2 pk{pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    reinterpret_cast<u32x2*>(y)[i] = pk;
  }
}

hipError_t launch_f32_to_f16(const float* x, uint16_t* y, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, y, n4);
  return hipGetLastError();
}

}  // namespace tsp
