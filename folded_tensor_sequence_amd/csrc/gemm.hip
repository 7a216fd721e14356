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
// Design: 256 threads = 4 waves in a 2x2 grid; a BM x BN tile (x NB weight
// matrices for the fused gate/up product) with BK = 64; global -> registers ->
// LDS double buffer with one barrier per K step; XOR-swizzled 128-byte LDS
// rows so both the 16-byte stores and the matrix-core operand reads are free
// of bank conflicts; 32x32x16 MFMA with the weight tile as the first operand
// so each lane ends up owning 4 consecutive output columns of one row.
// Blocks are remapped so that the tiles that share a weight block run on the
// same XCD (blocks are dealt round-robin to the 8 XCDs) and hit its L2.
#include "common.h"
#include "kernels.h"

namespace tsp {

enum { EPI_QKV = 0, EPI_RESID_BF16X = 1, EPI_RESID_F32 = 2, EPI_SWIGLU = 3 };

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
};

__device__ __forceinline__ float silu_f32(float z) {
  return z / (1.0f + __expf(-z));
}

template <int EPI>
__device__ __forceinline__ void epilogue4(const GemmArgs& a, int m, int n, const float* v,
                                          const float* v2) {
  if (m >= a.M || n >= a.N) return;
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
    const u32x2 xr = *reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(a.resid) + off);
    f32x4 o;
    o[0] = __uint_as_float(xr[0] << 16) + v[0];
    o[1] = __uint_as_float(xr[0] & 0xffff0000u) + v[1];
    o[2] = __uint_as_float(xr[1] << 16) + v[2];
    o[3] = __uint_as_float(xr[1] & 0xffff0000u) + v[3];
    *reinterpret_cast<f32x4*>(a.out + off) = o;
    if (a.out16 != nullptr) {
      u32x2 pk{pack_f16x2(o[0], o[1]), pack_f16x2(o[2], o[3])};
      *reinterpret_cast<u32x2*>(a.out16 + off) = pk;
    }
  } else if constexpr (EPI == EPI_RESID_F32) {
    const int64_t off = (int64_t)m * a.N + n;
    f32x4 r = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.resid) + off);
    f32x4 o;
    o[0] = r[0] + v[0];
    o[1] = r[1] + v[1];
    o[2] = r[2] + v[2];
    o[3] = r[3] + v[3];
    *reinterpret_cast<f32x4*>(a.out + off) = o;
  } else {  // EPI_SWIGLU: v = gate, v2 = up
    const int64_t off = (int64_t)m * a.N + n;
    u32x2 pk{pack_f16x2(silu_f32(v[0]) * v2[0], silu_f32(v[1]) * v2[1]),
             pack_f16x2(silu_f32(v[2]) * v2[2], silu_f32(v[3]) * v2[3])};
    *reinterpret_cast<u32x2*>(a.out16 + off) = pk;
  }
}

template <int BM, int BN, int NB, bool F16, bool CONVB, int EPI, int OCC>
__global__ __launch_bounds__(256, OCC) void gemm_kernel(GemmArgs a) {
  constexpr int BK = 64;
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int MB = WM / 32, NBL = WN / 32;
  constexpr int A_LD = BM / 32, B_LD = NB * BN / 32;
  constexpr int ROWB = BK * 2;
  constexpr int A_BYTES = BM * ROWB;
  constexpr int STAGE = (BM + NB * BN) * ROWB;
  __shared__ __align__(16) unsigned char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  // tile index: XCD-grouped so the blocks of one XCD cover consecutive tiles
  const int mtiles = (a.M + BM - 1) / BM;
  const int ntiles = mtiles * ((a.N + BN - 1) / BN);
  int logical;
  {
    const int bid = blockIdx.x, xcd = bid & 7, idx = bid >> 3;
    const int q = ntiles >> 3, rem = ntiles & 7;
    logical = xcd * q + (xcd < rem ? xcd : rem) + idx;
  }
  const int mt = logical % mtiles, nt = logical / mtiles;
  const int m0 = mt * BM, n0 = nt * BN;

  // global load assignment: row r_in (+32 i), 16-byte chunk cc of the 128-byte K slice
  const int r_in = tid >> 3, cc = tid & 7;
  const uint16_t* aptr[A_LD];
  const uint16_t* bptr[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    int m = m0 + r_in + 32 * i;
    m = m < a.M ? m : a.M - 1;
    aptr[i] = a.A + (int64_t)m * a.lda;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    const int row = r_in + 32 * i;
    const int which = row / BN;
    int n = n0 + (row - which * BN);
    n = n < a.N ? n : a.N - 1;
    const uint16_t* base = (NB == 2 && which == 1) ? a.B1 : a.B0;
    bptr[i] = base + (int64_t)n * a.ldb;
  }
  const int st_off = r_in * ROWB + ((cc ^ (r_in & 7)) << 4);

  u32x4 ra[A_LD], rb[B_LD];
  auto gload = [&](int kt) {
    const int k = kt * BK + cc * 8;
    const int sg = k / a.seg_len;
    const int kk = k - sg * a.seg_len;
    int j = sg;
    if (a.ring_rank >= 0) {
      j = a.ring_rank - sg;
      j = j < 0 ? j + a.nseg : j;
    }
    const int64_t aoff = (int64_t)j * a.a_seg_step + kk;
    const int64_t boff = (int64_t)j * a.b_seg_step + kk;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *reinterpret_cast<const u32x4*>(aptr[i] + aoff);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bptr[i] + boff);
  };
  auto lstore = [&](int stage) {
    unsigned char* sa = smem + stage * STAGE;
    unsigned char* sb = sa + A_BYTES;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *reinterpret_cast<u32x4*>(sa + st_off + i * 32 * ROWB) = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      u32x4 v = rb[i];
      if constexpr (CONVB) v = bf16x8_to_f16x8(v);
      *reinterpret_cast<u32x4*>(sb + st_off + i * 32 * ROWB) = v;
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

  const int lrow = lane & 31, lgrp = lane >> 5, lsw = lane & 7;
  const int nk = a.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const unsigned char* sa = smem + cur * STAGE;
    const unsigned char* sb = sa + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int pch = ((2 * ks + lgrp) ^ lsw) << 4;
      u32x4 af[MB], bf[NB][NBL];
#pragma unroll
      for (int z = 0; z < MB; ++z)
        af[z] = *reinterpret_cast<const u32x4*>(sa + (wm * WM + z * 32 + lrow) * ROWB + pch);
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int y = 0; y < NBL; ++y)
          bf[x][y] = *reinterpret_cast<const u32x4*>(sb + (x * BN + wn * WN + y * 32 + lrow) * ROWB + pch);
#pragma unroll
      for (int x = 0; x < NB; ++x)
#pragma unroll
        for (int y = 0; y < NBL; ++y)
#pragma unroll
          for (int z = 0; z < MB; ++z) {
            if constexpr (F16)
              acc[x][y][z] = mfma_f16(bf[x][y], af[z], acc[x][y][z]);
            else
              acc[x][y][z] = mfma_bf16(bf[x][y], af[z], acc[x][y][z]);
          }
    }
    if (kt + 1 < nk) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane owns row m = ... + lrow and columns n..n+3 per register quad
#pragma unroll
  for (int y = 0; y < NBL; ++y)
#pragma unroll
    for (int z = 0; z < MB; ++z) {
      const int m = m0 + wm * WM + z * 32 + lrow;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = n0 + wn * WN + y * 32 + 8 * q4 + 4 * lgrp;
        float v[4], v2[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = acc[0][y][z][4 * q4 + e];
          v2[e] = acc[NB - 1][y][z][4 * q4 + e];
        }
        epilogue4<EPI>(a, m, n, v, v2);
      }
    }
}

// --------------------------------------------------------------------------
// Host-side tile choice and launch
// --------------------------------------------------------------------------
template <int BM, int BN, int NB, bool F16, bool CONVB, int EPI, int OCC>
static hipError_t launch_tile(const GemmArgs& a, hipStream_t st) {
  const int mt = (a.M + BM - 1) / BM, nt = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, NB, F16, CONVB, EPI, OCC>), dim3(mt * nt), dim3(256), 0, st, a);
  return hipGetLastError();
}

static int tiles_of(int M, int N, int bm, int bn) {
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// Rough cost of a tile choice: waves of 256 CUs x tile work / relative
// per-CU efficiency of that tile shape.
static double tile_cost(int M, int N, int bm, int bn, int nb, double eff) {
  const int t = tiles_of(M, N, bm, bn);
  const int waves = (t + 255) / 256;
  return waves * (double)bm * bn * nb / eff;
}

template <bool F16, bool CONVB, int EPI>
static hipError_t launch_single(const GemmArgs& a, hipStream_t st) {
  const double big = tile_cost(a.M, a.N, 256, 256, 1, 1.0);
  const double small = tile_cost(a.M, a.N, 128, 128, 1, 0.8);
  if (big <= small) return launch_tile<256, 256, 1, F16, CONVB, EPI, 1>(a, st);
  return launch_tile<128, 128, 1, F16, CONVB, EPI, 2>(a, st);
}

static GemmArgs base_args(const Shape& s) {
  GemmArgs a{};
  a.s = s;
  a.ring_rank = -1;
  a.nseg = 1;
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
  return launch_single<false, false, EPI_QKV>(a, st);
}

hipError_t launch_oproj_gemm(const Shape& s, const uint16_t* o, const uint16_t* w_o,
                             const uint16_t* x_resid, float* out, uint16_t* out16, hipStream_t st) {
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
  a.resid = x_resid;
  return launch_single<true, true, EPI_RESID_BF16X>(a, st);
}

hipError_t launch_gateup_gemm(const Shape& s, const uint16_t* h16, const uint16_t* w_g,
                              const uint16_t* w_u, uint16_t* act, hipStream_t st) {
  GemmArgs a = base_args(s);
  a.A = h16;
  a.lda = s.h;
  a.B0 = w_g;
  a.B1 = w_u;
  a.ldb = s.h;
  a.M = s.M;
  a.N = s.F;
  a.K = s.h;
  a.seg_len = s.h;
  a.out16 = act;
  const double c1 = tile_cost(a.M, a.N, 256, 128, 2, 1.0);
  const double c2 = tile_cost(a.M, a.N, 128, 128, 2, 0.85);
  if (c1 <= c2) return launch_tile<256, 128, 2, true, true, EPI_SWIGLU, 1>(a, st);
  return launch_tile<128, 128, 2, true, true, EPI_SWIGLU, 1>(a, st);
}

hipError_t launch_down_gemm(const Shape& s, const uint16_t* act, const uint16_t* w_d,
                            const float* resid, float* y, hipStream_t st) {
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
  return launch_single<true, true, EPI_RESID_F32>(a, st);
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
