"""Seeded synthetic inputs for the one-rank TSP layer forward.

This module is shared by the oracle side and the GPU side and holds none of the
method's arithmetic: it only names the workload shapes and draws the random
tensors.  Every tensor is drawn in float32 from ``numpy.random.default_rng``
(PCG64) with ``standard_normal`` and rounded to bfloat16 with
round-to-nearest-even; the bit patterns (uint16) are what both sides consume.

Draw order (one generator per seed): X_full [B][S][h] ~ N(0,1), then
W_q [Hq*dh][h], W_k [Hkv*dh][h], W_v [Hkv*dh][h], W_o [h][Hq*dh],
W_g [F][h], W_u [F][h], W_d [h][F], all ~ N(0, sigma^2).

The weights are the unsharded nn.Linear-style matrices ([out][in]); how they
are cut into the D shards is the business of each side.
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = ["Dims", "Workload", "WORKLOADS", "workload", "f32_to_bf16_bits", "make_inputs", "make_custom",
           "make_grad"]


@dataclasses.dataclass(frozen=True)
class Dims:
    """Shape of one TSP layer forward as seen from one rank."""

    batch: int
    seq: int
    degree: int
    rank: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    partition: int = 0  # token partition: 0 zigzag, 1 striped

    def astuple(self):
        return dataclasses.astuple(self)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dims: Dims
    sigma: float
    seed: int
    about: str


# The five layer shapes.  Tiny is the small case the oracle finishes in
# seconds; the Llama-7B-like 8K layer is the headline one.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_d2", Dims(1, 256, 2, 0, 256, 4, 4, 64, 768), 0.02, 1,
                 "tiny layer, rank 0 of D=2, S=256, h=256, 4x64 MHA, ffn 768"),
        Workload("llama7b_s8k_d8", Dims(1, 8192, 8, 0, 4096, 32, 32, 128, 11008), 0.02, 2,
                 "Llama-7B-like layer, rank 0 of D=8, S=8192, h=4096, 32x128 MHA, SwiGLU ffn 11008"),
        Workload("llama3_8b_gqa_s16k_d8", Dims(2, 16384, 8, 3, 4096, 32, 8, 128, 14336), 0.02, 3,
                 "Llama-3-8B-like GQA layer, rank 3 of D=8, B=2, S=16384, h=4096, 32q/8kv x128, ffn 14336"),
        Workload("longctx_s128k_d8", Dims(1, 131072, 8, 7, 4096, 32, 8, 128, 14336), 0.02, 4,
                 "long-context GQA layer, rank 7 of D=8, S=131072, h=4096, 32q/8kv x128, ffn 14336"),
        Workload("wide70b_s32k_d8", Dims(1, 32768, 8, 0, 8192, 64, 8, 128, 28672), 0.015, 5,
                 "70B-like wide GQA layer, rank 0 of D=8, S=32768, h=8192, 64q/8kv x128, ffn 28672"),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    # NaN never occurs in these draws; round-to-nearest-even on the low 16 bits.
    rounding_bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding_bias) >> 16).astype(np.uint16)


def _draw(rng, shape, sigma):
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return f32_to_bf16_bits(a)


def make_inputs(dims: Dims, sigma: float, seed: int, x_rows: int | None = None) -> dict:
    """Draw the layer's inputs as bfloat16 bit patterns (uint16 arrays).

    ``x_rows`` limits the drawn X_full to the first ``x_rows`` positions of each
    sequence (the draw is still [B][S][h] in stream order, so the values of
    the kept rows do not depend on ``x_rows``); None keeps all S.
    """
    d = dims
    rng = np.random.default_rng(seed)
    out = {}
    # X is drawn sequence by sequence, row block by row block, to bound the
    # float32 scratch; the stream order equals one [B][S][h] draw.
    keep = d.seq if x_rows is None else int(x_rows)
    x = np.empty((d.batch, keep, d.hidden), dtype=np.uint16)
    block = 8192
    for b in range(d.batch):
        for s0 in range(0, d.seq, block):
            s1 = min(d.seq, s0 + block)
            blk = _draw(rng, (s1 - s0, d.hidden), 1.0)
            if s0 < keep:
                x[b, s0:min(s1, keep)] = blk[: min(s1, keep) - s0]
    out["x"] = x
    qd, kvd = d.n_q_heads * d.head_dim, d.n_kv_heads * d.head_dim
    out["w_q"] = _draw(rng, (qd, d.hidden), sigma)
    out["w_k"] = _draw(rng, (kvd, d.hidden), sigma)
    out["w_v"] = _draw(rng, (kvd, d.hidden), sigma)
    out["w_o"] = _draw(rng, (d.hidden, qd), sigma)
    out["w_g"] = _draw(rng, (d.ffn, d.hidden), sigma)
    out["w_u"] = _draw(rng, (d.ffn, d.hidden), sigma)
    out["w_d"] = _draw(rng, (d.hidden, d.ffn), sigma)
    return out


def make_custom(batch, seq, degree, rank, hidden, n_q_heads, n_kv_heads, head_dim, ffn,
                sigma=0.02, seed=0) -> tuple[Dims, dict]:
    """Convenience: dims plus inputs for an ad-hoc shape (parity sweeps)."""
    dims = Dims(batch, seq, degree, rank, hidden, n_q_heads, n_kv_heads, head_dim, ffn)
    return dims, make_inputs(dims, sigma, seed)



def make_grad(dims: Dims, seed: int, scale: float = 1.0) -> np.ndarray:
    """Upstream gradient dY of the layer output, float32 [B][S][h] ~ N(0, scale^2),
    from its own generator (seed + 7919, so it never repeats the input draw)."""
    rng = np.random.default_rng(seed + 7919)
    g = rng.standard_normal(size=(dims.batch, dims.seq, dims.hidden), dtype=np.float32)
    if scale != 1.0:
        g *= np.float32(scale)
    return g
