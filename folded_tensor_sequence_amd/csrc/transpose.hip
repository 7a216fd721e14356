// Transposes and type conversions feeding the backward GEMMs (gfx950).
//
// The backward of the gated MLP contracts over the token axis (weight
// gradients) and over the weights' output axis (input gradients).  The shard
// GEMM reads both operands K-contiguous, so those operands are transposed
// once into bfloat16 copies here.  A 64 x 64 tile goes through LDS: each
// thread reads 8 consecutive elements of one input row (16 bytes of a 16-bit
// input, 32 of a float32 one) and writes 8 consecutive elements of one output
// row (16 bytes), so a wave's reads and writes cover whole 128-byte runs.
#include "common.h"
#include "kernels.h"

namespace tsp {

namespace {

// Input element -> float (exact for bf16 and f16).
template <int TIN>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (TIN == TR_F32) {
    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  } else {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t x = w[e];
      if constexpr (TIN == TR_F16) {
        const f16x2 h = __builtin_bit_cast(f16x2, x);
        v[2 * e] = (float)h[0];
        v[2 * e + 1] = (float)h[1];
      } else {
        v[2 * e] = __uint_as_float(x << 16);
        v[2 * e + 1] = __uint_as_float(x & 0xffff0000u);
      }
    }
  }
}

__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

}  // namespace

// out[b][c][r] = bf16(in[b][r][c]) for r < R, c < C; out[b][c][r] = 0 for
// R <= r < Rp (Rp a multiple of 8: nothing at or past Rp is written, so an
// output block may sit inside a wider row).  Grid: (ceil(C / 64),
// ceil(Rp / 64), batches), 256 threads.
template <int TIN>
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const void* __restrict__ in, int64_t ld_in,
                                                             int64_t in_bstride, uint16_t* __restrict__ out,
                                                             int64_t ld_out, int64_t out_bstride, int R, int C,
                                                             int Rp) {
  __shared__ uint16_t tile[64][64 + 8];
  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
  const int64_t ib = (int64_t)blockIdx.z * in_bstride, ob = (int64_t)blockIdx.z * out_bstride;
  // read: thread (row i, chunk k) loads 8 elements of input row r0 + i
  const int k = tid & 7, i0 = tid >> 3;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int i = i0 + 32 * pass;
    const int r = r0 + i, c = c0 + 8 * k;
    float v[8];
    if (r < R && c < C) {
      load8<TIN>(in, ib + (int64_t)r * ld_in + c, v);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.0f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[i][8 * k + e] = to_bf16(v[e]);
  }
  __syncthreads();
  // write: thread (column j, chunk k) stores 8 elements of output row c0 + j
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int j = i0 + 32 * pass;
    const int c = c0 + j;
    if (c >= C || r0 + 8 * k >= Rp) continue;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)tile[8 * k + 2 * e][j] | ((uint32_t)tile[8 * k + 2 * e + 1][j] << 16);
    *reinterpret_cast<u32x4*>(out + ob + (int64_t)c * ld_out + r0 + 8 * k) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_transpose_bf16(int tin, const void* in, int64_t ld_in, int64_t in_bstride, uint16_t* out,
                                 int64_t ld_out, int64_t out_bstride, int R, int C, int Rp, int batches,
                                 hipStream_t st) {
  if (R < 0 || C < 0 || Rp < R || Rp % 8 != 0 || C % 8 != 0 || batches < 1) return hipErrorInvalidValue;
  if (Rp == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((Rp + 63) / 64), (unsigned)batches);
  switch (tin) {
    case TR_BF16:
      hipLaunchKernelGGL(transpose_bf16_kernel<TR_BF16>, grid, dim3(256), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C, Rp);
      break;
    case TR_F16:
      hipLaunchKernelGGL(transpose_bf16_kernel<TR_F16>, grid, dim3(256), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C, Rp);
      break;
    case TR_F32:
      hipLaunchKernelGGL(transpose_bf16_kernel<TR_F32>, grid, dim3(256), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C, Rp);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// out[b][r][c] = bf16(in[b][r][c]): 8 elements (one 16-byte store) per
// thread; grid (ceil(C / 8 / 64), min(R, 65535), batches), 64 threads, rows
// strided by the grid's y extent.
template <int TIN>
__global__ __launch_bounds__(64) void copy_bf16_kernel(const void* __restrict__ in, int64_t ld_in, int64_t in_bstride,
                                                       uint16_t* __restrict__ out, int64_t ld_out,
                                                       int64_t out_bstride, int R, int C) {
  const int c = (blockIdx.x * 64 + threadIdx.x) * 8;
  if (c >= C) return;
  const int64_t bz = blockIdx.z;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y) {
    float v[8];
    load8<TIN>(in, bz * in_bstride + r * ld_in + c, v);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (uint32_t)to_bf16(v[2 * e]) | ((uint32_t)to_bf16(v[2 * e + 1]) << 16);
    *reinterpret_cast<u32x4*>(out + bz * out_bstride + r * ld_out + c) = u32x4{w[0], w[1], w[2], w[3]};
  }
}

hipError_t launch_copy_bf16(int tin, const void* in, int64_t ld_in, int64_t in_bstride, uint16_t* out,
                            int64_t ld_out, int64_t out_bstride, int R, int C, int batches, hipStream_t st) {
  if (R < 0 || C < 0 || C % 8 != 0 || batches < 1 || batches > 65535) return hipErrorInvalidValue;
  if (R == 0 || C == 0) return hipSuccess;
  const dim3 grid((unsigned)((C / 8 + 63) / 64), (unsigned)(R < 65535 ? R : 65535), (unsigned)batches);
  switch (tin) {
    case TR_BF16:
      hipLaunchKernelGGL(copy_bf16_kernel<TR_BF16>, grid, dim3(64), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C);
      break;
    case TR_F16:
      hipLaunchKernelGGL(copy_bf16_kernel<TR_F16>, grid, dim3(64), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C);
      break;
    case TR_F32:
      hipLaunchKernelGGL(copy_bf16_kernel<TR_F32>, grid, dim3(64), 0, st, in, ld_in, in_bstride, out, ld_out,
                         out_bstride, R, C);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Elementwise float32 -> bf16 (round to nearest even), n a multiple of 4.
__global__ void f32_to_bf16_kernel(const float* __restrict__ x, uint16_t* __restrict__ y, int64_t n4) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n4; i += stride) {
    const f32x4 v = reinterpret_cast<const f32x4*>(x)[i];
    const uint32_t lo = (uint32_t)to_bf16(v[0]) | ((uint32_t)to_bf16(v[1]) << 16);
    const uint32_t hi = (uint32_t)to_bf16(v[2]) | ((uint32_t)to_bf16(v[3]) << 16);
    reinterpret_cast<u32x2*>(y)[i] = u32x2{lo, hi};
  }
}

hipError_t launch_f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, st, x, y, n4);
  return hipGetLastError();
}

}  // namespace tsp
