// Internal launchers of libtsp (host side).  Each returns the HIP error of
// its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace tsp {

// Kernel-choice override set through tsp_set_tuning (knob = tsp_tune_knob);
// -1 when none is set.
int tune_get(int knob);

hipError_t launch_zigzag_index(const Shape& s, int32_t* l2g, int32_t* g2s, hipStream_t st);
hipError_t launch_kv_reorder(const Shape& s, const uint16_t* gathered, uint16_t* knat,
                             uint16_t* vnat, hipStream_t st);

// Packed Q/K/V projection of src_rank's tokens (bf16 matrix cores).
hipError_t launch_qkv_gemm(const Shape& s, int src_rank, const uint16_t* x, const uint16_t* w_qkv,
                           uint16_t* q, uint16_t* kv_gathered, hipStream_t st);

// Largest split-K factor of the output and down projections; `partial` (float
// [kMaxSplit][M][h]) may be nullptr, which disables split-K.
constexpr int kMaxSplit = 4;

// Split-K factor planned for the output and down projections (both produce
// an M x h result with 256x128 tiles): 1 when the tiles already cover the 256
// CUs (224 or more), else up to kMaxSplit so that tiles x splits ~ 256.  The
// workspace holds split * M * h floats when it is > 1.
inline int gemm_split_plan(const Shape& s) {
  const int tiles = ((s.M + 255) / 256) * ((s.h + 127) / 128);
  if (tiles >= 224) return 1;
  int p = (256 + tiles - 1) / tiles;
  return p > kMaxSplit ? kMaxSplit : p;
}

// out = resid + O * W_o^T over the D shards' K-segments, where resid is
// x_resid (bf16) when given, else resid_f32 (float32), else nothing; also an
// f16 copy of out when out16 != nullptr.
hipError_t launch_oproj_gemm(const Shape& s, const uint16_t* o, const uint16_t* w_o,
                             const uint16_t* x_resid, const float* resid_f32, float* out, uint16_t* out16,
                             float* partial, hipStream_t st);

// act = silu(x Wg^T) * (x Wu^T): x f16 with f16 matrix cores (weights
// bf16 -> f16), or x bf16 (x_bf16) with bf16 matrix cores on the weights as
// given.  gu_keep (optional, float [2][M][F]): g = x Wg^T, then u = x Wu^T,
// as the epilogue receives them (for the backward).
hipError_t launch_gateup_gemm(const Shape& s, const uint16_t* x, bool x_bf16, const uint16_t* w_g,
                              const uint16_t* w_u, uint16_t* act, hipStream_t st, float* gu_keep = nullptr);

// y = resid + sum over ring steps of act_j W_d,j^T (resid may be nullptr).
hipError_t launch_down_gemm(const Shape& s, const uint16_t* act, const uint16_t* w_d,
                            const float* resid, float* y, float* partial, hipStream_t st);

// f32 -> f16 rounding copy (MLP input when it arrives as float32).
hipError_t launch_f32_to_f16(const float* x, uint16_t* y, int64_t n, hipStream_t st);

// ---- backward of the gated MLP ---------------------------------------------
// Input element types of launch_transpose_bf16.
enum { TR_BF16 = 0, TR_F16 = 1, TR_F32 = 2 };

// out[b][c][r] = bf16(in[b][r][c]) for r < R, c < C, zero for R <= r < Rp
// (Rp and C multiples of 8; rows 16-byte aligned; nothing past Rp written).
hipError_t launch_transpose_bf16(int tin, const void* in, int64_t ld_in, int64_t in_bstride, uint16_t* out,
                                 int64_t ld_out, int64_t out_bstride, int R, int C, int Rp, int batches,
                                 hipStream_t st);
hipError_t launch_f32_to_bf16(const float* x, uint16_t* y, int64_t n, hipStream_t st);

// dA = dy16 WdT^T (float32 [M][F]); WdT [F][h] bf16.
hipError_t launch_bwd_da(const Shape& s, const uint16_t* dy16, const uint16_t* wdT, float* da, hipStream_t st);
// dA = dy16 WdT^T in registers, with g and u kept from the forward (gu_keep,
// float [2][M][F]): the epilogue of launch_bwd_gu without dA's round trip
// through memory (act16 and dgu as there).
hipError_t launch_bwd_da_kept(const Shape& s, const uint16_t* dy16, const uint16_t* wdT, const float* gu_keep,
                              uint16_t* act16, uint16_t* dgu, hipStream_t st);
// g, u recomputed from x (f16, or bf16 when x_bf16); epilogue: act16 = a
// (bf16 [M][F]), dgu = dG | dU per shard (bf16 [M][D][2][F/D]).
hipError_t launch_bwd_gu(const Shape& s, const uint16_t* x, bool x_bf16, const uint16_t* w_g, const uint16_t* w_u,
                         const float* da, uint16_t* act16, uint16_t* dgu, hipStream_t st);
// dx = dx_resid + sum over ring steps of dGU_j WguT_j^T (dx_resid may be nullptr).
hipError_t launch_bwd_dx(const Shape& s, const uint16_t* dgu, const uint16_t* wguT, const float* dx_resid, float* dx,
                         float* partial, hipStream_t st);
// dW_down [D][h][F/D] = dyT aT^T; dW_gate, dW_up [F][h] = dguT xT^T.
hipError_t launch_bwd_dwd(const Shape& s, int m_pad, const uint16_t* dyT, const uint16_t* aT, float* dw_down,
                          hipStream_t st);
hipError_t launch_bwd_dwgu(const Shape& s, int m_pad, const uint16_t* dguT, const uint16_t* xT, float* dw_gate,
                           float* dw_up, hipStream_t st);

// Causal flash attention of the rank's queries over the all-gathered K/V
// (read in zigzag order through the position -> slot map, no reordered copy).
// Row blocks whose key range is long are cut into pieces along the keys
// (plan below); `partial` holds the pieces' state
// (attn_partial_bytes) and may be nullptr only when the plan has no pieces.
struct AttnPlan {
  int nwv, nst;     // waves per block, depth of the K/V ring
  int rb;           // rows per block (32 per wave)
  int nrb;          // row blocks per zigzag chunk
  int kt_max;       // key tiles (64 keys) per piece at most
  int pair;         // 1: earlier-chunk blocks run inside their later-chunk partner's last piece
  int64_t units;    // work groups of the attention kernel
  int pieces;       // pieces of split blocks, summed over the block list
  int split_rows;   // rb x (number of split blocks)
};
AttnPlan attn_plan(const Shape& s);
// The default plan for blocks of nwv waves (4 or 8).
AttnPlan attn_plan_shape(const Shape& s, int nwv);
size_t attn_partial_bytes(const Shape& s);
// lse (optional, float [B][Hq][T]): each row's log2 softmax normaliser of
// the scaled scores, for the backward pass.
hipError_t launch_flash_attn(const Shape& s, const uint16_t* q, const uint16_t* kv_gathered, uint16_t* o,
                             float* partial, hipStream_t st, float* lse = nullptr);

// ---- backward of the attention ----------------------------------------------
// Projections (bf16 matrix cores): q = x Wq^T (Wq: the Q rows of every shard of
// W_QKV [D][nqkv_s][h], read in place; q f16 [B][Hq][T][dh]);
// dO = dh16 WoT^T (f16 [M][Hq*dh]); dW_O [D][h][Hq/D dh] = dhT oT^T;
// dx = dx_resid + G WqkvT^T (G [M][D nqkv_s] bf16, ring order over the
// shards); dW_QKV [D nqkv_s][h] = gT xT^T.
hipError_t launch_q_gemm(const Shape& s, const uint16_t* x, const uint16_t* w_qkv, uint16_t* q, hipStream_t st);
hipError_t launch_attn_bwd_do(const Shape& s, const uint16_t* dh16, const uint16_t* woT, uint16_t* dout,
                              hipStream_t st);
hipError_t launch_attn_bwd_dwo(const Shape& s, int m_pad, const uint16_t* dhT, const uint16_t* oT, float* dw_o,
                               hipStream_t st);
hipError_t launch_attn_bwd_dx(const Shape& s, const uint16_t* g16, const uint16_t* wqkvT, const float* dx_resid,
                              float* dx, float* partial, hipStream_t st);
hipError_t launch_attn_bwd_dwqkv(const Shape& s, int m_pad, const uint16_t* gT, const uint16_t* xT, float* dw_qkv,
                                 hipStream_t st);
// The same backward products with the weight read as stored (K-major, no
// transposed copy): dA = dy16 W_down (also with launch_bwd_da_kept's
// epilogue), dx = dx_resid + ring sum of dG_j
// W_gate,j + dU_j W_up,j, dO = dh16 W_O, dx = dx_resid + G W_QKV (ring
// order).  kmajor_ok(s, use) tells whether the variant applies to the shape
// (K segments whole multiples of 64, operands within 32-bit offsets); the
// launchers return hipErrorInvalidValue, launching nothing, when it does not.
enum { KMAJ_DA = 0, KMAJ_DX_MLP = 1, KMAJ_DO = 2, KMAJ_DX_ATTN = 3 };
bool kmajor_ok(const Shape& s, int use);
hipError_t launch_bwd_da_kmajor(const Shape& s, const uint16_t* dy16, const uint16_t* w_down, float* da,
                                hipStream_t st);
hipError_t launch_bwd_da_kept_kmajor(const Shape& s, const uint16_t* dy16, const uint16_t* w_down,
                                     const float* gu_keep, uint16_t* act16, uint16_t* dgu, hipStream_t st);
hipError_t launch_bwd_dx_kmajor(const Shape& s, const uint16_t* dgu, const uint16_t* w_g, const uint16_t* w_u,
                                const float* dx_resid, float* dx, float* partial, hipStream_t st);
hipError_t launch_attn_bwd_do_kmajor(const Shape& s, const uint16_t* dh16, const uint16_t* w_o, uint16_t* dout,
                                     hipStream_t st);
hipError_t launch_attn_bwd_dx_kmajor(const Shape& s, const uint16_t* g16, const uint16_t* w_qkv,
                                     const float* dx_resid, float* dx, float* partial, hipStream_t st);
// out[b][r][c] = bf16(in[b][r][c]) (bit copy for a bf16 input), r < R, c < C
// (C a multiple of 8, rows 16-byte aligned).
hipError_t launch_copy_bf16(int tin, const void* in, int64_t ld_in, int64_t in_bstride, uint16_t* out,
                            int64_t ld_out, int64_t out_bstride, int R, int C, int batches, hipStream_t st);

// From the rank's Q (f16 [B][Hq][T][dh]), the all-gathered K/V, the
// recomputed output O and its gradient dO (f16 [B][T][Hq*dh]) and the
// forward's row normalisers lse ([B][Hq][T]): delta = rowsum(dO * O)
// ([B][Hq][T], written), dq (float [B][T][Hq*dh], unscaled Q space) and the
// rank's contribution to every key's K/V gradient, dkv_send (float
// [D dst][D shard][K|V][B][T][Hkv/D*dh], grouped by the keys' owner ranks).
// partial: attn_partial_bytes of scratch (pieces of split row blocks).
hipError_t launch_attn_bwd_core(const Shape& s, const uint16_t* q, const uint16_t* kv_gathered, const uint16_t* o,
                                const uint16_t* dout, const float* lse, float* delta, float* dq, float* dkv_send,
                                float* partial, hipStream_t st);

}  // namespace tsp
