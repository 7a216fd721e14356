"""Storage-rounding model of the layer: the error floor of an f16 evaluation.

TEST INFRASTRUCTURE ONLY, under the same rules as ``tsp_oracle``: only
``tests/`` may import it; the HIP library never routes through it and shares
no code with it.

The layer of ``tsp_oracle`` (h = x + Attn(x), y = h + SwiGLU-MLP(h), Zyphra
TSP article, "How to Fold a Book") is evaluated in float64, except that chosen
intermediates are rounded to IEEE binary16 (round to nearest even) where a
matrix-core implementation with 16-bit operands has to store them:

    "qkv"  the Q, K and V projections;
    "p"    the softmax probabilities fed to P V (the row sum is taken over the
           rounded values, so normalisation stays consistent with P V);
    "o"    the attention output before the output projection;
    "h16"  the copy of h that feeds the MLP (h itself stays wide for the
           residual);
    "act"  the SwiGLU activation silu(h Wg^T) * (h Wu^T) fed to the down
           projection.

Everything else (accumulation, softmax arithmetic, residual adds) stays
float64, so with every point enabled the result is the error any correct
f16-storage evaluation carries at the least; with none enabled it is the
oracle itself.  This sets the expected error floor for each workload and
tells which intermediate dominates it.
"""
from __future__ import annotations

import math

import numpy as np

from . import tsp_oracle as orc

POINTS = ("qkv", "p", "o", "h16", "act")


def f16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to binary16 (round to nearest even) and back."""
    return np.asarray(a, dtype=np.float64).astype(np.float16).astype(np.float64)


def rank_rows_rounded(inputs: dict, dims, b: int, rows, points=POINTS, kv=None, weights=None) -> np.ndarray:
    """y for local rows ``rows`` of sequence b, with the storage points in
    ``points`` rounded to binary16.  ``kv``/``weights`` as in
    ``tsp_oracle.rank_rows_forward``."""
    unknown = set(points) - set(POINTS)
    if unknown:
        raise ValueError(f"unknown rounding points {sorted(unknown)}")
    R = (lambda name, a: f16(a) if name in points else a)
    B, S, D, r, h, Hq, Hkv, dh, F = orc._dims(dims)
    rows = np.asarray(rows, dtype=np.int64)
    g = orc.local_to_global(S, D, r, orc._part(dims))[rows]
    if weights is None:
        weights = {n: orc.bf16_bits_to_f64(inputs[n]) for n in ("w_q", "w_o", "w_g", "w_u", "w_d")}
    n_keys = int(g.max()) + 1
    if kv is None:
        kv = orc.project_kv(inputs, dims, b, n_keys)
    k, v = R("qkv", kv[0][:n_keys]), R("qkv", kv[1][:n_keys])
    x = orc.bf16_bits_to_f64(inputs["x"][b, g])
    q = R("qkv", x @ weights["w_q"].T)
    o = np.empty((len(rows), Hq * dh))
    group = Hq // Hkv
    masked = np.arange(n_keys)[None, :] > g[:, None]
    for i in range(Hq):
        kvh = i // group
        s = (q[:, i * dh:(i + 1) * dh] @ k[:, kvh * dh:(kvh + 1) * dh].T) / math.sqrt(dh)
        s[masked] = -np.inf
        p = R("p", np.exp(s - s.max(axis=1, keepdims=True)))
        o[:, i * dh:(i + 1) * dh] = (p @ v[:, kvh * dh:(kvh + 1) * dh]) / p.sum(axis=1, keepdims=True)
    hres = x + R("o", o) @ weights["w_o"].T
    hm = R("h16", hres)
    act = R("act", orc.silu(hm @ weights["w_g"].T) * (hm @ weights["w_u"].T))
    return hres + act @ weights["w_d"].T


# --------------------------------------------------------------------------- #
# Backward of the gated MLP: bfloat16 storage points
# --------------------------------------------------------------------------- #
BWD_POINTS = ("dy", "act", "dgu", "xw")


def bf16(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (round to nearest even) and back, via
    float32 (exact for every bfloat16 value; float64 -> float32 rounding
    first is a double rounding only for values within 2^-29 relative of a
    bfloat16 tie, which random data does not hit)."""
    f = np.asarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def mlp_backward_rounded(x: np.ndarray, w_g: np.ndarray, w_u: np.ndarray, w_d: np.ndarray, dy: np.ndarray,
                         points=BWD_POINTS, x_f16: bool = False) -> dict:
    """The gated MLP's backward (``tsp_backward.mlp_backward``) in float64 with
    the storage points in ``points`` rounded to bfloat16 where a matrix-core
    implementation with 16-bit operands keeps them:

        "dy"   the upstream gradient fed to dA = dy Wd and dWd = dy^T a;
        "act"  the activation a = silu(g) u fed to dWd;
        "dgu"  dG and dU fed to dx and to dWg, dWu;
        "xw"   the MLP input fed to dWg, dWu.

    ``x_f16``: the recomputation of g and u sees x rounded to binary16 (an
    input handed over as float32)."""
    unknown = set(points) - set(BWD_POINTS)
    if unknown:
        raise ValueError(f"unknown rounding points {sorted(unknown)}")
    R = (lambda name, a: bf16(a) if name in points else a)
    xg = f16(x) if x_f16 else x
    g, u = xg @ w_g.T, xg @ w_u.T
    s = 1.0 / (1.0 + np.exp(-g))
    a = g * s * u
    dyr = R("dy", dy)
    da = dyr @ w_d
    du, dg = R("dgu", da * g * s), R("dgu", da * u * (s + g * s * (1.0 - s)))
    xw = R("xw", x)
    return {"dx": dg @ w_g + du @ w_u, "dw_g": dg.T @ xw, "dw_u": du.T @ xw, "dw_d": dyr.T @ R("act", a)}
