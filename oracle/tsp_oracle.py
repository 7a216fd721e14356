"""Plain CPU float64 oracle for one rank's share of a TSP transformer-layer forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this module.
The HIP library never routes through it, and it shares no code with the HIP
path: its only common ground with the GPU side is the seeded input generator
(``synth``), which holds no arithmetic of the method.

What is computed, and where the pages define it
-----------------------------------------------
Tensor-and-Sequence Parallelism (TSP) folds tensor and sequence parallelism
onto one device axis of size D: every rank keeps 1/D of every weight matrix and
1/D of the tokens (Zyphra TSP article on ai-trends.today, "Zyphra Introduces
Tensor and Sequence Parallelism (TSP)...", section "How to Fold a Book"; the
aivizor.me news post "Zyphra представила TSP-схему шардирования...", third
paragraph).  The two schedules it uses -- attention by iterating over packed
weight shards with a K/V all-gather and zigzag reorder, and a gated MLP by a
weight ring -- are exact re-partitionings of the unsharded layer: column splits
followed by row splits sum to the full product and attention splits by heads
(bowenzhou.top "张量并行", section "机制：行切与列切"; r007.github.io
"Распределенное обучение", section "Тензорный параллелизм").  The zigzag
partition only permutes tokens.  Hence the oracle is the plain definition:

    layer_rank_rows   the unsharded layer in float64 from the bfloat16 inputs,
                      sliced to the rank's zigzag rows (the reference result);
    tsp_schedule      the TSP schedule itself over all D virtual ranks (shard
                      iteration, simulated all-gather + zigzag reorder, per-shard
                      attention, MLP weight ring), used to show that the method
                      reproduces the unsharded layer.

Readings where the pages are silent (each one is listed in the design notes):
  * layer form: h = x + Attn(x), y = h + MLP(h); no norm, rotary embedding,
    bias or dropout (the pages name only "attention" then "gated MLP");
  * attention scale 1/sqrt(head_dim), causal mask inclusive (key <= query);
  * gated MLP = SwiGLU: (silu(x Wg^T) * (x Wu^T)) Wd^T, silu(z) = z/(1+e^-z);
  * zigzag: rank r holds chunks r and 2D-1-r of 2D equal chunks, local order
    chunk r first; GQA q-head i reads kv-head floor(i*Hkv/Hq);
  * striped (the pages only name it beside zigzag): position g on rank
    g mod D at local row g div D, token by token;
  * shard j = contiguous head group j (q-heads [j*Hq/D, (j+1)*Hq/D), kv-heads
    likewise) and MLP rows/cols [j*F/D, (j+1)*F/D);
  * ring order: at step s rank r uses MLP shard (r - s) mod D;
  * batches are independent sequences, each split the same way.

Query rows are processed in blocks only to bound memory; every output row is
computed exactly as the definition states (no reassociation inside a row
beyond what BLAS does for a dot product).

Every function below has at least one pin in ``tests/test_oracle_pins.py``
that does not re-run this module's own formula.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bf16_bits_to_f64",
    "ZIGZAG",
    "STRIPED",
    "local_to_global",
    "global_to_slot",
    "causal_pairs",
    "causal_attention",
    "silu",
    "swiglu_mlp",
    "layer_rank_rows",
    "project_kv",
    "rank_rows_forward",
    "qkv_rows",
    "mlp_block",
    "tsp_schedule",
    "algorithmic_flops",
]


# --------------------------------------------------------------------------- #
# Input decoding
# --------------------------------------------------------------------------- #
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------- #
# Token partitions.
# Zigzag (TSP article, "How to Fold a Book": K/V are collected and reordered
# with a zigzag partition to balance causal work; r007.github.io
# "Распределенное обучение", "Параллелизм по контексту: Ring Attention против
# Ulysses", item 1: zigzag or striped token partitions spread the causal tiles
# evenly).  Exact form: the sequence is cut into 2D equal chunks and rank r
# holds chunk r followed by chunk 2D-1-r.
# Striped (the other partition that passage names): position g belongs to
# rank g mod D, as its local row g div D.
# --------------------------------------------------------------------------- #
ZIGZAG, STRIPED = 0, 1


def local_to_global(S: int, D: int, r: int, partition: int = ZIGZAG) -> np.ndarray:
    """Global sequence position of each of rank r's S/D local rows."""
    if S % (2 * D) or not 0 <= r < D:
        raise ValueError("need S % 2D == 0 and 0 <= r < D")
    if partition == STRIPED:
        return np.array([t * D + r for t in range(S // D)], dtype=np.int64)
    if partition != ZIGZAG:
        raise ValueError(f"unknown partition {partition}")
    c = S // (2 * D)
    first = [r * c + i for i in range(c)]
    second = [(2 * D - 1 - r) * c + i for i in range(c)]
    return np.array(first + second, dtype=np.int64)


def global_to_slot(S: int, D: int, partition: int = ZIGZAG) -> np.ndarray:
    """For each global position g, its slot rank*(S/D) + local_row in a
    rank-major all-gathered buffer (inverse of the per-rank local_to_global)."""
    T = S // D
    slot = np.full(S, -1, dtype=np.int64)
    for r in range(D):
        for t, g in enumerate(local_to_global(S, D, r, partition)):
            slot[g] = r * T + t
    return slot


def causal_pairs(S: int, D: int, r: int, partition: int = ZIGZAG) -> int:
    """Number of causal (query, key) pairs, key <= query, for rank r's rows
    (brute-force count over the rows' global positions)."""
    return int(sum(int(g) + 1 for g in local_to_global(S, D, r, partition)))


# --------------------------------------------------------------------------- #
# Attention (causal softmax attention of one head)
# --------------------------------------------------------------------------- #
def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                     scale: float | None = None, block: int = 256) -> np.ndarray:
    """o[i] = sum_{j <= q_pos[i]} softmax_j(q[i].k[j] * scale) v[j].

    q [n][dh] float64 with global positions q_pos[n]; k, v [>= max(q_pos)+1][dh].
    The softmax subtracts the row maximum before exponentiating (exact up to
    rounding; it only keeps exp() in range).
    """
    q = np.asarray(q, dtype=np.float64)
    dh = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for i0 in range(0, q.shape[0], block):
        i1 = min(q.shape[0], i0 + block)
        pos = q_pos[i0:i1]
        nk = int(pos.max()) + 1
        s = (q[i0:i1] @ k[:nk].T) * scale
        masked = np.arange(nk)[None, :] > pos[:, None]
        s[masked] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[i0:i1] = p @ v[:nk]
    return out


# --------------------------------------------------------------------------- #
# Gated MLP (SwiGLU form)
# --------------------------------------------------------------------------- #
def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z / (1 + exp(-z)), evaluated without overflow for large |z|."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_mlp(x: np.ndarray, w_g: np.ndarray, w_u: np.ndarray, w_d: np.ndarray) -> np.ndarray:
    """(silu(x Wg^T) * (x Wu^T)) Wd^T with nn.Linear-style [out][in] weights."""
    return (silu(x @ w_g.T) * (x @ w_u.T)) @ w_d.T


# --------------------------------------------------------------------------- #
# The unsharded layer, sliced to the rank's rows
# --------------------------------------------------------------------------- #
def _dims(d):
    return (d.batch, d.seq, d.degree, d.rank, d.hidden, d.n_q_heads, d.n_kv_heads,
            d.head_dim, d.ffn)


def _part(d) -> int:
    return getattr(d, "partition", ZIGZAG)


def project_kv(inputs: dict, dims, b: int, n_keys: int, block: int = 4096):
    """K = X_b[:n_keys] W_k^T, V = X_b[:n_keys] W_v^T in float64."""
    w_k = bf16_bits_to_f64(inputs["w_k"])
    w_v = bf16_bits_to_f64(inputs["w_v"])
    kvd = w_k.shape[0]
    k = np.empty((n_keys, kvd))
    v = np.empty((n_keys, kvd))
    for s0 in range(0, n_keys, block):
        s1 = min(n_keys, s0 + block)
        xb = bf16_bits_to_f64(inputs["x"][b, s0:s1])
        k[s0:s1] = xb @ w_k.T
        v[s0:s1] = xb @ w_v.T
    return k, v


def rank_rows_forward(inputs: dict, dims, b: int, rows: np.ndarray, kv=None,
                      weights=None) -> dict:
    """Layer outputs for local rows ``rows`` of sequence b on rank dims.rank.

    Returns float64 arrays [len(rows)][...]: 'o' (attention heads, before the
    output projection), 'attn' (O W_o^T), 'h' (x + attn), 'mlp', 'y' (h + mlp).
    ``kv`` optionally holds precomputed (K, V) for at least max(global)+1 keys.
    """
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    rows = np.asarray(rows, dtype=np.int64)
    g = local_to_global(S, D, r, _part(dims))[rows]
    if weights is None:
        weights = {n: bf16_bits_to_f64(inputs[n]) for n in ("w_q", "w_o", "w_g", "w_u", "w_d")}
    n_keys = int(g.max()) + 1
    if kv is None:
        kv = project_kv(inputs, dims, b, n_keys)
    k, v = kv
    x = bf16_bits_to_f64(inputs["x"][b, g])
    q = x @ weights["w_q"].T
    o = np.empty((len(rows), Hq * dh))
    group = Hq // Hkv
    for i in range(Hq):
        kvh = i // group  # == floor(i * Hkv / Hq)
        o[:, i * dh:(i + 1) * dh] = causal_attention(
            q[:, i * dh:(i + 1) * dh], k[:, kvh * dh:(kvh + 1) * dh],
            v[:, kvh * dh:(kvh + 1) * dh], g)
    attn = o @ weights["w_o"].T
    hres = x + attn
    mlp = swiglu_mlp(hres, weights["w_g"], weights["w_u"], weights["w_d"])
    return {"o": o, "attn": attn, "h": hres, "mlp": mlp, "y": hres + mlp, "x": x}


def qkv_rows(inputs: dict, dims, b: int, rows, rank=None) -> dict:
    """Q, K, V projections X W^T of local rows ``rows`` of sequence b on rank
    ``rank`` (default dims.rank), float64, unsharded head order."""
    r = dims.rank if rank is None else rank
    g = local_to_global(dims.seq, dims.degree, r, _part(dims))[np.asarray(rows, dtype=np.int64)]
    x = bf16_bits_to_f64(inputs["x"][b, g])
    return {n: x @ bf16_bits_to_f64(inputs["w_" + n]).T for n in ("q", "k", "v")}


def mlp_block(inputs: dict, x: np.ndarray) -> np.ndarray:
    """x + SwiGLU-MLP(x) for float64 rows x [n][h] (the MLP half of the layer)."""
    w_g, w_u, w_d = (bf16_bits_to_f64(inputs[n]) for n in ("w_g", "w_u", "w_d"))
    return x + swiglu_mlp(x, w_g, w_u, w_d)


def layer_rank_rows(inputs: dict, dims, rows=None) -> dict:
    """Unsharded float64 layer on every sequence, sliced to rank dims.rank.

    ``rows`` selects local rows (same for every sequence); None = all S/D.
    Each returned array is [B][len(rows)][...].
    """
    T = dims.seq // dims.degree
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    weights = {n: bf16_bits_to_f64(inputs[n]) for n in ("w_q", "w_o", "w_g", "w_u", "w_d")}
    per_b = [rank_rows_forward(inputs, dims, b, rows, weights=weights) for b in range(dims.batch)]
    return {key: np.stack([p[key] for p in per_b]) for key in per_b[0]}


# --------------------------------------------------------------------------- #
# The TSP schedule over all D virtual ranks (no communication: exchanges are
# array copies).  TSP article, "How to Fold a Book": attention iterates over
# weight shards -- the owner of shard j hands its packed W_Q/W_K/W_V/W_O to
# every rank, each rank projects its own tokens, K and V are all-gathered and
# reordered with the zigzag partition before attention; the gated MLP passes
# gate/up/down shards around a ring and each rank accumulates partial outputs
# locally, so no all-reduce is needed.
# --------------------------------------------------------------------------- #
def tsp_schedule(inputs: dict, dims) -> np.ndarray:
    """Returns y for every rank: [D][B][S/D][h] float64."""
    B, S, D, _r, h, Hq, Hkv, dh, F = _dims(dims)
    T = S // D
    hq_s, hkv_s, f_s = Hq // D, Hkv // D, F // D
    w_q, w_k, w_v, w_o, w_g, w_u, w_d = (bf16_bits_to_f64(inputs[n]) for n in
                                         ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d"))
    x_all = bf16_bits_to_f64(inputs["x"])
    l2g = [local_to_global(S, D, r, _part(dims)) for r in range(D)]
    slot = global_to_slot(S, D, _part(dims))
    x_loc = [x_all[:, l2g[r]] for r in range(D)]          # each [B][T][h]
    attn = [np.zeros((B, T, h)) for _ in range(D)]
    group = Hq // Hkv
    for j in range(D):
        # packed attention shard j (head group j)
        qrows = slice(j * hq_s * dh, (j + 1) * hq_s * dh)
        kvrows = slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        wq_j, wk_j, wv_j = w_q[qrows], w_k[kvrows], w_v[kvrows]
        wo_j = w_o[:, qrows]
        q_j = [x_loc[r] @ wq_j.T for r in range(D)]
        # all-gather: rank-major [D*T] per sequence, then reorder to sequence order
        k_gath = np.concatenate([x_loc[r] @ wk_j.T for r in range(D)], axis=1)
        v_gath = np.concatenate([x_loc[r] @ wv_j.T for r in range(D)], axis=1)
        k_nat = k_gath[:, slot]
        v_nat = v_gath[:, slot]
        for r in range(D):
            o_j = np.empty((B, T, hq_s * dh))
            for b in range(B):
                for i in range(hq_s):
                    kvh = (j * hq_s + i) // group - j * hkv_s
                    o_j[b, :, i * dh:(i + 1) * dh] = causal_attention(
                        q_j[r][b, :, i * dh:(i + 1) * dh],
                        k_nat[b, :, kvh * dh:(kvh + 1) * dh],
                        v_nat[b, :, kvh * dh:(kvh + 1) * dh], l2g[r])
            attn[r] += o_j @ wo_j.T                      # row-split partial sum
    y = np.empty((D, B, T, h))
    for r in range(D):
        hres = x_loc[r] + attn[r]
        acc = np.zeros_like(hres)
        for s in range(D):                                # MLP weight ring
            j = (r - s) % D
            rows = slice(j * f_s, (j + 1) * f_s)
            acc += swiglu_mlp(hres, w_g[rows], w_u[rows], w_d[:, rows])
        y[r] = hres + acc
    return y


# --------------------------------------------------------------------------- #
# Work accounting (for throughput figures): 2*M*N*K per GEMM and
# 4*dh per (query, key) causal pair per query head; masked pairs, softmax and
# elementwise work are not counted.
# --------------------------------------------------------------------------- #
def algorithmic_flops(dims, rows_per_seq=None) -> dict:
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    T = S // D
    g = local_to_global(S, D, r, _part(dims))
    if rows_per_seq is not None:
        g = g[np.asarray(rows_per_seq)]
    m = B * len(g)
    pairs = B * int((g + 1).sum())
    qkv = 2.0 * m * (Hq + 2 * Hkv) * dh * h
    o = 2.0 * m * Hq * dh * h
    att = 4.0 * dh * Hq * pairs
    mlp = 2.0 * m * 3 * F * h
    return {"qkv": qkv, "o": o, "attn": att, "mlp": mlp, "total": qkv + o + att + mlp}
