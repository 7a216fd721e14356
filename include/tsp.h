/* tsp.h -- C ABI of libtsp: one rank's share of a Tensor-and-Sequence-Parallel
 * (TSP) transformer-layer forward on one AMD Instinct MI355X (gfx950).
 *
 * What TSP computes (Zyphra TSP article on ai-trends.today, "Zyphra Introduces
 * Tensor and Sequence Parallelism (TSP)...", section "How to Fold a Book"):
 * one device axis of size D carries both tensor and sequence parallelism, so
 * rank r keeps 1/D of every weight matrix and 1/D of the tokens.  Attention
 * iterates over packed weight shards {W_Q, W_K, W_V, W_O}: every rank
 * projects its own tokens with shard j, K and V are all-gathered, reordered
 * with the zigzag partition and fed to causal attention; the output
 * projection of shard j is a row split whose partials are summed locally.
 * The gated MLP runs as a ring over gate/up/down weight shards; each rank
 * accumulates its partial outputs locally and the sequence never moves.
 *
 * This library computes the per-rank work with all D weight shards already
 * resident in device memory (no collectives).  The layer is read as
 *     h = x + Attn(x),   y = h + MLP(h),
 *     MLP(h) = (silu(h Wg^T) * (h Wu^T)) Wd^T,  silu(z) = z / (1 + e^-z),
 * causal attention with scale 1/sqrt(head_dim) and keys k <= query q, no
 * normalisation, rotary embedding, bias or dropout.
 *
 * Token partitions (r007.github.io "Распределенное обучение", section
 * "Параллелизм по контексту: Ring Attention против Ulysses", item 1, names
 * zigzag and striped partitions as the ways to balance causal tiles):
 *   zigzag (default, the one the TSP article uses): the sequence of S
 *     positions is cut into 2D chunks of c = S/(2D); rank r holds chunk r then
 *     chunk 2D-1-r (local row order), i.e. local row t has global position
 *     r*c + t for t < c and (2D-1-r)*c + (t-c) otherwise;
 *   striped: local row t of rank r has global position t*D + r (position g
 *     lives on rank g mod D at row g div D).  GQA: q-head i reads kv-head floor(i*Hkv/Hq).  Shard j is head
 * group j: q-heads [j*Hq/D, (j+1)*Hq/D), kv-heads [j*Hkv/D, (j+1)*Hkv/D), and
 * MLP rows/columns [j*F/D, (j+1)*F/D).  The MLP ring at step s uses shard
 * (r - s) mod D.
 *
 * General rules for every entry point
 *   - Tensor pointers are DEVICE memory owned by the caller, 16-byte aligned.
 *     16-bit tensors are passed as uint16_t bit patterns: "bf16" = bfloat16,
 *     "f16" = IEEE half.  All index arithmetic is 64-bit.
 *   - Every call is asynchronous on `stream` (NULL = the default stream); it
 *     never synchronises and never allocates device memory.
 *   - Arguments are validated before anything is launched.  The return value
 *     is TSP_OK (0) or a negative tsp_status; tsp_last_error() then returns a
 *     thread-local message.  A failed launch returns TSP_ERR_HIP.
 *   - Inputs are read-only; outputs are overwritten in full.
 *   - Overlapping calls on different streams must not share outputs or
 *     workspace.
 */
#ifndef TSP_H_
#define TSP_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Layer shape as seen from one rank.
 *   batch      B >= 1 independent sequences, each zigzag-split the same way
 *   seq        S, total positions per sequence;   S % (2*degree) == 0
 *   degree     D >= 1, size of the TSP axis
 *   rank       r in [0, D)
 *   hidden     h, h % 64 == 0
 *   n_q_heads  Hq, n_kv_heads Hkv:  Hq % D == 0, Hkv % D == 0, Hq % Hkv == 0
 *   head_dim   dh in {64, 128}
 *   ffn        F, F % 64 == 0 and (F/D) % 8 == 0
 *   partition  TSP_PARTITION_ZIGZAG (0) or TSP_PARTITION_STRIPED (1); a
 *              zero-initialised struct means zigzag
 * Derived: T = S/D local rows per sequence, c = S/(2D), M = B*T, F_s = F/D,
 *   kmax = one past the largest position rank r attends to: (2D - r)*c for
 *   zigzag, (T - 1)*D + r + 1 for striped;
 *   kmax_pad = kmax rounded up to a multiple of 64.
 */
typedef struct {
  int32_t batch, seq, degree, rank, hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  int32_t partition;
} tsp_dims_t;

typedef enum { TSP_PARTITION_ZIGZAG = 0, TSP_PARTITION_STRIPED = 1 } tsp_partition;

/* Return codes.  Every validation failure has a code of its own; the text
 * from tsp_last_error() names the argument and the rule it broke. */
typedef enum {
  TSP_OK = 0,
  TSP_ERR_INVALID_ARG = -1,  /* argument outside its documented set (selector, src_rank, ...) */
  TSP_ERR_UNSUPPORTED = -2,  /* valid TSP shape the library does not handle (head_dim, index range) */
  TSP_ERR_WORKSPACE = -3,    /* ws too small (see tsp_workspace_bytes) */
  TSP_ERR_HIP = -4,          /* HIP runtime error (no device, launch failure) */
  TSP_ERR_NULL_POINTER = -5, /* a required pointer (or dims) is NULL */
  TSP_ERR_MISALIGNED = -6,   /* a tensor pointer is not 16-byte aligned */
  TSP_ERR_BATCH = -10,       /* batch < 1 */
  TSP_ERR_DEGREE = -11,      /* degree < 1 */
  TSP_ERR_RANK = -12,        /* rank (or src_rank) not in [0, degree) */
  TSP_ERR_SEQ = -13,         /* seq not a positive multiple of 2*degree */
  TSP_ERR_HEADS = -14,       /* a head count < 1 or not a multiple of degree */
  TSP_ERR_GQA = -15,         /* n_q_heads not a multiple of n_kv_heads */
  TSP_ERR_HIDDEN = -16,      /* hidden not a positive multiple of 64 */
  TSP_ERR_FFN = -17,         /* ffn not a positive multiple of 64, or ffn/degree not a multiple of 8 */
  TSP_ERR_PARTITION = -18,   /* unknown token partition */
  TSP_ERR_DTYPE = -19,       /* unknown tsp_dtype */
  TSP_ERR_KMAX = -20,        /* kmax outside [0, seq] */
  TSP_ERR_SCRATCH = -21      /* problem larger than the library's fixed scratch array */
} tsp_status;

/* Element types of tensors whose type the caller chooses. */
typedef enum { TSP_BF16 = 0, TSP_F16 = 1, TSP_F32 = 2 } tsp_dtype;

/* Selectors for tsp_workspace_bytes. */
typedef enum {
  TSP_FN_ATTN = 1,       /* tsp_attn_fwd workspace */
  TSP_FN_MLP = 2,        /* tsp_mlp_ring_fwd workspace */
  TSP_FN_LAYER = 3,      /* tsp_layer_fwd workspace */
  TSP_FN_KV_NATURAL = 4, /* size of the kv_natural output of tsp_kv_reorder */
  TSP_FN_KV_GATHERED = 5, /* size of the kv_gathered buffer */
  TSP_FN_MLP_BWD = 6,    /* tsp_mlp_ring_bwd workspace */
  TSP_FN_ATTN_BWD = 7,   /* tsp_attn_bwd workspace */
  TSP_FN_ATTN_BWD_PROJ = 8, /* tsp_attn_bwd_proj workspace */
  TSP_FN_DKV = 9,        /* size of tsp_attn_bwd's dkv_send output */
  TSP_FN_ATTN_KEEP = 10, /* tsp_attn_fwd_keep workspace */
  TSP_FN_ATTN_BWD_KEPT = 11, /* tsp_attn_bwd_kept workspace */
  TSP_FN_LSE = 12,       /* size of tsp_attn_fwd_keep's lse_keep output */
  TSP_FN_MLP_BWD_KEPT = 13, /* tsp_mlp_ring_bwd_kept workspace */
  TSP_FN_GU = 14         /* size of tsp_mlp_ring_fwd_keep's gu_keep output */
} tsp_fn;

/* Maps of the partition dims->partition selects, as described above (TSP
 * article, "How to Fold a Book": K/V are reordered with a zigzag partition
 * that balances causal work across ranks; r007.github.io "Распределенное
 * обучение", section "Параллелизм по контексту: Ring Attention против
 * Ulysses", item 1, for zigzag and striped partitions).
 *   local_to_global  int32 [T]: global position of rank dims->rank's row t.
 *   global_to_slot   int32 [S] or NULL: for each global position g, the slot
 *                    rank*T + t that holds it in a rank-major all-gather.
 * Both maps are exact integers. */
int tsp_zigzag_index(const tsp_dims_t* dims, int32_t* local_to_global,
                     int32_t* global_to_slot, hipStream_t stream);

/* Packed per-shard Q/K/V projection of one rank's tokens (TSP article, "How
 * to Fold a Book": each rank applies the broadcast W_Q/W_K/W_V of shard j to
 * its own tokens).  Computes X_src * W_qkv,j^T for every shard j with bf16
 * matrix cores and float32 accumulation, rounding results to f16.
 *   src_rank     rank whose tokens x_shard holds (its partition rows)
 *   x_shard      bf16 [B][T][h], local row order of src_rank
 *   w_qkv        bf16 [D][(Hq/D + 2*Hkv/D)*dh][h]: shard j's rows are its
 *                Hq/D q-heads, then its Hkv/D k-heads, then its v-heads,
 *                dh rows each, in nn.Linear [out][in] order
 *   q_out        f16 [B][Hq][T][dh] or NULL (then Q is not stored)
 *   kv_gathered  f16 [D_shard][D_src][2][B][T][Hkv/D*dh]: the all-gather
 *                destination; this call writes only the src_rank slots
 *                (index 0 of the [2] axis is K, 1 is V).
 * The library uses this for its own rank inside tsp_attn_fwd/tsp_layer_fwd;
 * a caller simulating the other ranks' all-gather contributions calls it
 * once per other rank. */
int tsp_qkv_proj(const tsp_dims_t* dims, int32_t src_rank, const uint16_t* x_shard,
                 const uint16_t* w_qkv, uint16_t* q_out, uint16_t* kv_gathered,
                 hipStream_t stream);

/* Reorder of the gathered K/V into natural sequence order through the
 * partition's position -> slot map (TSP article, "How to Fold a Book": the
 * all-gathered K and V are reordered with the zigzag partition before
 * attention).  Bit-exact 16-bit copy of every key position g < kmax; the
 * positions [kmax, kmax_pad) are zero-filled.
 *   kv_gathered  f16, layout of tsp_qkv_proj, all D_src slots filled
 *   kmax         number of leading positions to reorder: 0 means the rank's
 *                own kmax (above); otherwise 1 <= kmax <= seq (else
 *                TSP_ERR_KMAX).  kmax_pad = kmax rounded up to 64.
 *   kv_natural   f16, 4*Hkv*B*kmax_pad*dh bytes (TSP_FN_KV_NATURAL gives it
 *                for kmax = 0):
 *                K part  [Hkv][B][kmax_pad][dh]   (key-major rows)
 *                V part  [Hkv][B][dh][kmax_pad]   (transposed: dh-major)
 *                the V part starts right after the K part; the kv-head
 *                index is the global one, j*Hkv/D + (head within shard j). */
int tsp_kv_reorder(const tsp_dims_t* dims, const uint16_t* kv_gathered,
                   uint16_t* kv_natural, int32_t kmax, hipStream_t stream);

/* Attention half of the layer on rank dims->rank:
 *     out = residual + sum_j O_j W_O,j^T     (residual NULL: out = the sum),
 * O_j = causal attention of the rank's queries (q-heads of shard j) at their
 * partition positions over the K/V of shard j in natural sequence order (TSP
 * article, "How to Fold a Book": every rank projects its tokens with the
 * broadcast W_Q/W_K/W_V/W_O of shard j, K/V are all-gathered and put in
 * sequence order, then attention; the head split with a row-split output
 * projection sums exactly: bowenzhou.top "张量并行", section "机制：行切与列切").
 * The attention kernel applies the partition's position -> slot map while it
 * loads K/V tiles from kv_gathered, so no reordered copy is made.
 *   x_local      bf16 [B][T][h]
 *   w_qkv        bf16, layout of tsp_qkv_proj;  w_o bf16 [D][h][Hq/D*dh]
 *                (shard j = W_o columns of its q-heads)
 *   kv_gathered  in: the other ranks' slots; out: this rank's slots
 *   residual     float32 [B][T][h] or NULL (the attention branch alone)
 *   out          float32 [B][T][h]; may alias residual
 *   ws           device workspace of >= tsp_workspace_bytes(dims, TSP_FN_ATTN)
 * Precision: Q/K/V, softmax probabilities and O are f16 with float32
 * accumulation and float32 online softmax; W_o is read as bf16 and rounded
 * to f16 for the matrix cores. */
int tsp_attn_fwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                 const uint16_t* w_o, uint16_t* kv_gathered, const float* residual, float* out,
                 void* ws, size_t ws_bytes, hipStream_t stream);

/* Gated-MLP weight ring on rank dims->rank (TSP article, "How to Fold a
 * Book": gate/up/down shards travel around a ring, partial outputs are
 * accumulated locally, no all-reduce; the column/row split sums exactly,
 * bowenzhou.top "张量并行", section "机制：行切与列切"):
 *     y = residual + sum_{s=0}^{D-1} (silu(x Wg_j^T) * (x Wu_j^T)) Wd_j^T,  j = (r - s) mod D
 * (residual NULL: y = the sum alone).
 *   x        [B][T][h] of type x_dtype: TSP_BF16 (bf16 matrix cores on x as
 *            given), TSP_F16, or TSP_F32 (rounded to f16 for the matrix
 *            cores; values must lie in the f16 range)
 *   w_gate, w_up  bf16 [D][F/D][h] (= [F][h]);  w_down bf16 [D][h][F/D]
 *   residual float32 [B][T][h] or NULL
 *   y        float32 [B][T][h]; may alias residual or x
 *   ws       >= tsp_workspace_bytes(dims, TSP_FN_MLP) bytes */
int tsp_mlp_ring_fwd(const tsp_dims_t* dims, const void* x, int32_t x_dtype,
                     const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                     const float* residual, float* y, void* ws, size_t ws_bytes,
                     hipStream_t stream);

/* Backward of the gated-MLP weight ring on rank dims->rank: the gradients of
 *     m = sum_{s=0}^{D-1} (silu(x Wg_j^T) * (x Wu_j^T)) Wd_j^T,  j = (r - s) mod D
 * for the upstream gradient dy = dL/dm of the rank's own tokens.  The TSP
 * article presents TSP for training ("Zyphra Introduces Tensor and Sequence
 * Parallelism (TSP)...", opening paragraph and "What you need to know") but
 * describes only the forward schedule; this is its transpose.  The shards go
 * round the ring again, each carrying an accumulator of its weight
 * gradients: a rank adds its own tokens' contribution to the shard it holds,
 * so every accumulator reaches its owner with the sum over all ranks; the
 * input gradient stays local and sums over the shards (the transpose of the
 * column/row split: bowenzhou.top "张量并行", section "机制：行切与列切").
 * With all D shards resident, this call computes the rank's input gradient
 * and its contribution to every shard's weight gradients:
 *     dA_j = dy Wd_j,  dU_j = dA_j * silu(g_j),  dG_j = dA_j * u_j * silu'(g_j),
 *     dx   = dx_residual + sum_s (dG_j Wg_j + dU_j Wu_j)   (ring order),
 *     dWg_j = dG_j^T x,  dWu_j = dU_j^T x,  dWd_j = dy^T (silu(g_j) * u_j),
 * with g_j = x Wg_j^T, u_j = x Wu_j^T recomputed, silu'(z) = s (1 + z (1 - s)),
 * s = 1 / (1 + e^-z).
 *   x            [B][T][h] MLP input of type x_dtype (as in tsp_mlp_ring_fwd)
 *   dy           float32 [B][T][h]
 *   w_gate, w_up, w_down   bf16, layouts of tsp_mlp_ring_fwd
 *   dx_residual  float32 [B][T][h] or NULL, added to dx (pass dy for the
 *                residual branch of y = x + MLP(x))
 *   dx           float32 [B][T][h]; may alias dy or dx_residual
 *   dw_gate, dw_up  float32 [D][F/D][h] (= [F][h]): this rank's contribution
 *   dw_down      float32 [D][h][F/D]: this rank's contribution
 *   ws           >= tsp_workspace_bytes(dims, TSP_FN_MLP_BWD) bytes
 * Precision: dy and the gradients dA, dG, dU, the activation a and x enter
 * the matrix cores as bf16 (bfloat16 keeps float32's range, which gradients
 * need); the recomputation of g and u runs as in the forward; float32
 * accumulation and float32 outputs. */
int tsp_mlp_ring_bwd(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const float* dy,
                     const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                     const float* dx_residual, float* dx, float* dw_gate, float* dw_up, float* dw_down,
                     void* ws, size_t ws_bytes, hipStream_t stream);

/* The MLP backward with the forward's gate and up values kept instead of
 * recomputed (the other side of the recompute-or-keep choice the pages leave
 * open; tsp_mlp_ring_bwd recomputes): tsp_mlp_ring_fwd_keep is
 * tsp_mlp_ring_fwd that also hands g_j = x Wg_j^T and u_j = x Wu_j^T of every
 * shard (float32, as its matrix cores accumulated them) to the caller, and
 * tsp_mlp_ring_bwd_kept is tsp_mlp_ring_bwd from them (its outputs bit for
 * bit under the default kernel choice, where the forward's gate/up product
 * and the backward's recomputation are the same kernel): the product
 * dA = dy Wd forms a, dG and dU as it finishes, so neither
 * the recomputing gate/up product nor dA's trip through memory runs.  The
 * kept tensor costs 8 M F bytes per layer (86 MiB at the 8K layer).
 * tsp_mlp_ring_fwd_keep arguments: those of tsp_mlp_ring_fwd, and
 *   gu_keep  float32 [2][B][T][F] out (tsp_workspace_bytes(dims, TSP_FN_GU)
 *            bytes): g of all F columns, then u (shard j's columns are
 *            j F/D .. (j + 1) F/D - 1, the rows of w_gate and w_up); must
 *            not overlap any other argument
 *   ws       >= tsp_workspace_bytes(dims, TSP_FN_MLP) bytes
 * tsp_mlp_ring_bwd_kept arguments: those of tsp_mlp_ring_bwd, plus gu_keep
 * from tsp_mlp_ring_fwd_keep on the same dims, x, x_dtype and weights (read
 * only; x still feeds dW_gate and dW_up), and
 *   ws       >= tsp_workspace_bytes(dims, TSP_FN_MLP_BWD_KEPT) bytes */
int tsp_mlp_ring_fwd_keep(const tsp_dims_t* dims, const void* x, int32_t x_dtype,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          const float* residual, float* y, float* gu_keep, void* ws, size_t ws_bytes,
                          hipStream_t stream);
int tsp_mlp_ring_bwd_kept(const tsp_dims_t* dims, const void* x, int32_t x_dtype, const float* dy,
                          const uint16_t* w_gate, const uint16_t* w_up, const uint16_t* w_down,
                          const float* gu_keep, const float* dx_residual, float* dx, float* dw_gate,
                          float* dw_up, float* dw_down, void* ws, size_t ws_bytes, hipStream_t stream);

/* Backward of the attention on rank dims->rank, in the two parts that the
 * K/V-gradient reduce-scatter separates.  The TSP article gives the forward
 * schedule only ("How to Fold a Book": each rank projects its tokens with
 * every shard, K and V are all-gathered, and each rank attends with its own
 * queries over all keys); its transpose, for the gradient dh of the rank's
 * tokens at the attention branch's output (h = x + Attn(x)):
 *   1. tsp_attn_bwd: the rank recomputes Q = x W_Q^T and the attention
 *      output O with its row normalisers (activation recomputation), forms
 *      dO = dh W_O and, for every head, the softmax gradient
 *          P = softmax(Q K^T / sqrt(dh)) (causal), dP = dO V^T,
 *          dS = P * (dP - rowsum(dO * O)),
 *          dQ = dS K / sqrt(dh),  dK = dS^T Q / sqrt(dh),  dV = P^T dO;
 *      dK and dV of every key (all D ranks' tokens) are its contribution to
 *      the reduce-scatter that returns each key's sum over all ranks' queries
 *      to the key's owner.  Also its tokens' share of dW_O = dh^T O.
 *   2. tsp_attn_bwd_proj, after the reduce-scatter: with dQ and the summed
 *      dK, dV of its own tokens, the input gradient
 *          dx = dx_residual + dQ W_Q + dK W_K + dV W_V
 *      and its tokens' share of the packed dW_Q, dW_K, dW_V (summed at the
 *      shard owners, the transpose of the weight broadcast).
 * tsp_attn_bwd arguments:
 *   x_local, w_qkv, w_o   as in tsp_attn_fwd
 *   kv_gathered  f16, the all-gathered K/V (layout of tsp_attn_fwd), every
 *                rank's slot filled (read only)
 *   dh           float32 [B][T][h], the gradient at h of the rank's tokens
 *   dq           float32 [B][T][Hq*dh] out: dL/dQ of the rank's queries
 *                (Q = x W_Q^T, before the 1/sqrt(dh) scale)
 *   dkv_send     float32 [D dst][D shard][K|V][B][T][Hkv/D*dh] out
 *                (tsp_workspace_bytes(dims, TSP_FN_DKV) bytes): the rank's
 *                contribution to the K and V gradients of every key, grouped
 *                by the key's owner rank dst (so block dst is the piece the
 *                reduce-scatter sends to rank dst) at the owner's local row;
 *                zero for keys no query of this rank sees
 *   dw_o         float32 [D][h][Hq/D*dh] out (the layout of w_o): this rank's
 *                tokens' share of dW_O
 *   ws           >= tsp_workspace_bytes(dims, TSP_FN_ATTN_BWD) bytes
 * tsp_attn_bwd_proj arguments:
 *   x_local, w_qkv  as in tsp_attn_fwd
 *   dq           float32 [B][T][Hq*dh] (from tsp_attn_bwd)
 *   dkv_own      float32 [D shard][K|V][B][T][Hkv/D*dh]: the sum over all D
 *                ranks of their dkv_send blocks for this rank
 *   dx_residual  float32 [B][T][h] or NULL, added to dx (pass dh for the
 *                residual branch of h = x + Attn(x))
 *   dx           float32 [B][T][h] out; may alias dx_residual
 *   dw_qkv       float32 [D][(Hq/D + 2 Hkv/D)*dh][h] out (the layout of
 *                w_qkv): this rank's tokens' share
 *   ws           >= tsp_workspace_bytes(dims, TSP_FN_ATTN_BWD_PROJ) bytes
 * Precision: Q, K, V, O, dO, P and dS enter the matrix cores as f16 (as in
 * the forward; P and dS lie in [-1, 1] times dP's range); dh, O (for dW_O),
 * the gradient rows and x enter the projection GEMMs as bf16; float32
 * softmax, accumulation and outputs.  Both calls are deterministic (fixed
 * summation order, no atomics). */
int tsp_attn_bwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv, const uint16_t* w_o,
                 const uint16_t* kv_gathered, const float* dh, float* dq, float* dkv_send, float* dw_o, void* ws,
                 size_t ws_bytes, hipStream_t stream);
int tsp_attn_bwd_proj(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv, const float* dq,
                      const float* dkv_own, const float* dx_residual, float* dx, float* dw_qkv, void* ws,
                      size_t ws_bytes, hipStream_t stream);

/* The attention backward with the forward's activations kept instead of
 * recomputed (the other side of the recompute-or-keep choice the pages leave
 * open; tsp_attn_bwd recomputes): tsp_attn_fwd_keep is tsp_attn_fwd that
 * also hands its Q, its attention output O and each row's softmax
 * normaliser to the caller, and tsp_attn_bwd_kept is part 1 of the backward
 * (tsp_attn_bwd's outputs, bit for bit) from them, skipping the
 * recomputation of Q and of the attention (about a fifth of part 1's time at
 * the 8K layer).  The kept tensors cost 2 M Hq dh 2 + B Hq T 4 bytes per
 * layer (about 16 MiB per layer at the 8K layer, 256 MiB at 128K).
 * tsp_attn_fwd_keep arguments: those of tsp_attn_fwd, and
 *   q_keep    f16 [B][Hq][T][dh] out: Q of the rank's tokens (all heads)
 *   o_keep    f16 [B][T][Hq*dh] out: the attention output before W_O
 *   lse_keep  float32 [B][Hq][T] out (tsp_workspace_bytes(dims, TSP_FN_LSE)
 *             bytes): log2 of each row's softmax normaliser of the scaled
 *             scores, so P = 2^(s log2(e) / sqrt(dh) - lse)
 *   ws        >= tsp_workspace_bytes(dims, TSP_FN_ATTN_KEEP) bytes
 * tsp_attn_bwd_kept arguments: those of tsp_attn_bwd without x_local and
 * w_qkv, plus q_keep, o_keep and lse_keep from tsp_attn_fwd_keep on the same
 * dims and K/V (read only), and
 *   ws        >= tsp_workspace_bytes(dims, TSP_FN_ATTN_BWD_KEPT) bytes */
int tsp_attn_fwd_keep(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                      const uint16_t* w_o, uint16_t* kv_gathered, const float* residual, float* out,
                      uint16_t* q_keep, uint16_t* o_keep, float* lse_keep, void* ws, size_t ws_bytes,
                      hipStream_t stream);
int tsp_attn_bwd_kept(const tsp_dims_t* dims, const uint16_t* w_o, const uint16_t* kv_gathered,
                      const uint16_t* q_keep, const uint16_t* o_keep, const float* lse_keep, const float* dh,
                      float* dq, float* dkv_send, float* dw_o, void* ws, size_t ws_bytes, hipStream_t stream);

/* Whole layer on rank dims->rank: h = x + Attn(x), y = h + MLP(h), with the
 * argument layouts of tsp_attn_fwd and tsp_mlp_ring_fwd.  h stays float32;
 * its f16 copy feeds the MLP matrix cores.
 *   y   float32 [B][T][h]
 *   ws  >= tsp_workspace_bytes(dims, TSP_FN_LAYER) bytes */
int tsp_layer_fwd(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                  const uint16_t* w_o, const uint16_t* w_gate, const uint16_t* w_up,
                  const uint16_t* w_down, uint16_t* kv_gathered, float* y, void* ws,
                  size_t ws_bytes, hipStream_t stream);

/* tsp_layer_fwd without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It allocates nothing: its workspace is
 * a fixed array of TSP_SCRATCH_BYTES inside the library, one per GPU, held
 * until the process ends.  Layers needing more workspace than that
 * (tsp_workspace_bytes(dims, TSP_FN_LAYER) > TSP_SCRATCH_BYTES) return
 * TSP_ERR_SCRATCH before anything is launched.  Nothing in the array has to
 * start at zero (every piece is written before it is read).  Every call on
 * one GPU uses the same array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  The first call
 * on a device looks the array's device address up (no allocation). */
#define TSP_SCRATCH_BYTES (128u * 1024u * 1024u)
int tsp_layer_fwd_noalloc(const tsp_dims_t* dims, const uint16_t* x_local, const uint16_t* w_qkv,
                          const uint16_t* w_o, const uint16_t* w_gate, const uint16_t* w_up,
                          const uint16_t* w_down, uint16_t* kv_gathered, float* y, hipStream_t stream);

/* Bytes of workspace (or of a buffer) named by fn for these dims; 0 if the
 * dims are invalid (tsp_last_error says why). */
size_t tsp_workspace_bytes(const tsp_dims_t* dims, int32_t fn);

/* Kernels of the layer, for tsp_profile_kernel. */
typedef enum {
  TSP_K_NONE = 0,
  TSP_K_QKV = 1,     /* packed Q/K/V projection GEMM */
  TSP_K_REORDER = 2, /* zigzag K/V reorder */
  TSP_K_ATTN = 3,    /* causal flash attention */
  TSP_K_OPROJ = 4,   /* output projection GEMM (+ residual) */
  TSP_K_GATEUP = 5,  /* MLP gate/up GEMM with the SwiGLU epilogue */
  TSP_K_DOWN = 6,    /* MLP down-projection ring GEMM (+ residual) */
  TSP_K_ATTN_BWD = 7, /* attention backward core: Delta, dQ (+ merge), dK/dV kernels */
  TSP_K_COUNT = 8
} tsp_kernel_id;

/* Live timing of one kernel: after tsp_profile_kernel(id, n) the next n
 * launches of kernel `id` made by this thread (through any entry point) are
 * bracketed by a pair of HIP events recorded on the launch stream.  The
 * events are created here, once, not inside the timed calls, as timing-only
 * events (no system-scope fence, so recording them does not write back the
 * caches between the kernels).  id = TSP_K_NONE stops and releases them.
 * Not for use while a HIP graph is being captured. */
int tsp_profile_kernel(int32_t kernel_id, int32_t max_launches);

/* Waits for the recorded events of the current profile and returns the number
 * of bracketed launches and their summed duration in milliseconds; the
 * profile stays armed for the same kernel with its counters reset. */
int tsp_profile_result(int32_t* launches, float* total_ms);

/* Kernel-choice overrides, for tests and tuning only.  The default dispatch
 * depends on the shape alone; an override set here replaces one decision for
 * every later launch in the process until it is reset (value < 0).  Not
 * synchronised with launches in flight on other threads.
 *   TSP_TUNE_GEMM_*    GEMM configuration index (see the GEMM source)
 *   TSP_TUNE_SPLIT_*   split-K factor 1..4 of the output / down projection
 *   TSP_TUNE_ATTN_SHAPE  4: 4 waves x 2 K/V stages, 8: 8 waves x 3 stages
 *   TSP_TUNE_ATTN_PAIR   0 or 1: pair the two halves' row blocks or not
 *   TSP_TUNE_ATTN_PIECES target number of attention work units (> 0)
 *   TSP_TUNE_BWD_WEIGHTS 1: the backward calls multiply by transposed copies
 *                        of the weights (held in their workspace) instead of
 *                        reading the weights as stored; the workspace size
 *                        (tsp_workspace_bytes) depends on this knob */
typedef enum {
  TSP_TUNE_GEMM_QKV = 0,
  TSP_TUNE_GEMM_OPROJ = 1,
  TSP_TUNE_GEMM_GATEUP = 2,
  TSP_TUNE_GEMM_DOWN = 3,
  TSP_TUNE_SPLIT_OPROJ = 4,
  TSP_TUNE_SPLIT_DOWN = 5,
  TSP_TUNE_ATTN_SHAPE = 6,
  TSP_TUNE_ATTN_PAIR = 7,
  TSP_TUNE_ATTN_PIECES = 8,
  TSP_TUNE_BWD_WEIGHTS = 9,
  TSP_TUNE_COUNT = 10
} tsp_tune_knob;

int tsp_set_tuning(int32_t knob, int32_t value);

/* Thread-local text describing the last non-zero return on this thread. */
const char* tsp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TSP_H_ */
