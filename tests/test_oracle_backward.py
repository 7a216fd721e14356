"""Pins for the CPU backward oracle (``oracle/tsp_backward.py``) against
things other than itself: PyTorch float64 autograd of an independent forward,
central finite differences, brute-force loops, and the TSP backward schedule
reproducing the unsharded gradients.  CPU only."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import synth
from oracle import tsp_backward as bwd
from oracle import tsp_oracle as orc

TINY = [  # (B, S, D, r, h, Hq, Hkv, dh, F): non-square, GQA, B = 2
    (2, 8, 2, 0, 6, 4, 2, 2, 10),
    (1, 16, 4, 1, 8, 4, 4, 4, 16),
    (2, 12, 3, 2, 6, 6, 3, 2, 12),
]


def _torch_layer(inp, d, wt, xt):
    """The layer forward in torch float64 ops (an independent implementation)."""
    B, S = d.batch, d.seq
    rep = d.n_q_heads // d.n_kv_heads
    q = (xt @ wt["w_q"].T).view(B, S, d.n_q_heads, d.head_dim).transpose(1, 2)
    k = (xt @ wt["w_k"].T).view(B, S, d.n_kv_heads, d.head_dim).transpose(1, 2)
    v = (xt @ wt["w_v"].T).view(B, S, d.n_kv_heads, d.head_dim).transpose(1, 2)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k.repeat_interleave(rep, 1), v.repeat_interleave(rep, 1), is_causal=True)
    o = o.transpose(1, 2).reshape(B, S, -1)
    hres = xt + o @ wt["w_o"].T
    return hres + (torch.nn.functional.silu(hres @ wt["w_g"].T) * (hres @ wt["w_u"].T)) @ wt["w_d"].T


def _setup(shape, seed=31, sigma=0.4):
    d = synth.Dims(*shape)
    inp = synth.make_inputs(d, sigma, seed)
    dy = synth.make_grad(d, seed).astype(np.float64)
    return d, inp, dy


@pytest.mark.parametrize("shape", TINY)
def test_layer_backward_matches_torch_autograd(shape):
    d, inp, dy = _setup(shape)
    got = bwd.layer_backward(inp, d, dy)
    wt = {n: torch.from_numpy(orc.bf16_bits_to_f64(inp[n])).requires_grad_(True) for n in bwd.WEIGHTS}
    xt = torch.from_numpy(orc.bf16_bits_to_f64(inp["x"])).requires_grad_(True)
    y = _torch_layer(inp, d, wt, xt)
    (y * torch.from_numpy(dy)).sum().backward()
    np.testing.assert_allclose(got["dx"], xt.grad.numpy(), rtol=1e-10, atol=1e-11)
    for n in bwd.WEIGHTS:
        np.testing.assert_allclose(got["d" + n], wt[n].grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=n)


def test_layer_backward_finite_differences():
    # directional derivatives of L = sum(y * dy) by central differences of
    # the torch forward, for x and every weight
    d, inp, dy = _setup(TINY[0], seed=32)
    got = bwd.layer_backward(inp, d, dy)
    base = {n: orc.bf16_bits_to_f64(inp[n]) for n in bwd.WEIGHTS}
    base["x"] = orc.bf16_bits_to_f64(inp["x"])
    rng = np.random.default_rng(5)

    def loss(vals):
        wt = {n: torch.from_numpy(vals[n]) for n in bwd.WEIGHTS}
        return float((_torch_layer(inp, d, wt, torch.from_numpy(vals["x"])) * torch.from_numpy(dy)).sum())

    eps = 1e-6
    for n in ("x",) + bwd.WEIGHTS:
        v = rng.standard_normal(base[n].shape)
        plus = dict(base, **{n: base[n] + eps * v})
        minus = dict(base, **{n: base[n] - eps * v})
        fd = (loss(plus) - loss(minus)) / (2 * eps)
        an = float((got["dx" if n == "x" else "d" + n] * v).sum())
        assert fd == pytest.approx(an, rel=1e-6, abs=1e-8), n


def test_mlp_backward_matches_bruteforce():
    rng = np.random.default_rng(7)
    n, h, F = 3, 5, 7
    x, dy = rng.standard_normal((n, h)), rng.standard_normal((n, h))
    wg, wu, wd = rng.standard_normal((F, h)), rng.standard_normal((F, h)), rng.standard_normal((h, F))
    got = bwd.mlp_backward(x, wg, wu, wd, dy)
    dx = np.zeros((n, h))
    dwg, dwu, dwd = np.zeros((F, h)), np.zeros((F, h)), np.zeros((h, F))
    for i in range(n):
        for f in range(F):
            g = sum(x[i, k] * wg[f, k] for k in range(h))
            u = sum(x[i, k] * wu[f, k] for k in range(h))
            s = 1.0 / (1.0 + math.exp(-g))
            a = g * s * u
            da = sum(dy[i, o] * wd[o, f] for o in range(h))
            for o in range(h):
                dwd[o, f] += dy[i, o] * a
            dg = da * u * (s + g * s * (1 - s))
            du = da * g * s
            for k in range(h):
                dx[i, k] += dg * wg[f, k] + du * wu[f, k]
                dwg[f, k] += dg * x[i, k]
                dwu[f, k] += du * x[i, k]
    for key, want in (("dx", dx), ("dw_g", dwg), ("dw_u", dwu), ("dw_d", dwd)):
        np.testing.assert_allclose(got[key], want, rtol=1e-12, atol=1e-12, err_msg=key)


def test_attention_backward_matches_torch_autograd_on_subset_positions():
    # queries at scattered positions (a rank's zigzag rows) against all keys
    rng = np.random.default_rng(8)
    nk, dh, dv = 20, 6, 4
    k, v = rng.standard_normal((nk, dh)), rng.standard_normal((nk, dv))
    pos = np.array([0, 1, 9, 10, 18, 19])
    q, do = rng.standard_normal((len(pos), dh)), rng.standard_normal((len(pos), dv))
    dq, dk, dvv = bwd.attention_backward(q, k, v, pos, do, block=4)
    qt, kt, vt = (torch.from_numpy(a).requires_grad_(True) for a in (q, k, v))
    s = qt @ kt.T / math.sqrt(dh)
    s = s.masked_fill(torch.from_numpy(np.arange(nk)[None, :] > pos[:, None]), float("-inf"))
    (torch.softmax(s, dim=1) @ vt * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, qt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dk, kt.grad.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dvv, vt.grad.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(dk[pos.max() + 1:] == 0) and np.all(dvv[pos.max() + 1:] == 0)


@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
def test_tsp_backward_schedule_equals_unsharded(shape, partition):
    d, inp, dy = _setup(shape, seed=33)
    d = dataclasses.replace(d, partition=partition)
    want = bwd.layer_backward(inp, d, dy)
    got = bwd.tsp_backward_schedule(inp, d, dy)
    np.testing.assert_allclose(got["dx"], want["dx"], rtol=1e-11, atol=1e-12)
    for n in bwd.WEIGHTS:
        np.testing.assert_allclose(got["d" + n], want["d" + n], rtol=1e-11, atol=1e-12, err_msg=n)


@pytest.mark.parametrize("shape", TINY)
def test_rank_mlp_shares_sum_to_the_unsharded_gradients(shape):
    # each rank's MLP-ring share (its tokens, all shards in ring order): the
    # input gradient equals the unsharded one on its rows; the weight
    # gradients summed over ranks equal the unsharded MLP's
    d, inp, dy = _setup(shape, seed=34)
    B, S, D = d.batch, d.seq, d.degree
    wg, wu, wd = (orc.bf16_bits_to_f64(inp[n]) for n in ("w_g", "w_u", "w_d"))
    rng = np.random.default_rng(9)
    h_all = rng.standard_normal((B, S, d.hidden))          # any MLP input
    tot = {k: 0.0 for k in ("dw_g", "dw_u", "dw_d")}
    for r in range(D):
        l2g = orc.local_to_global(S, D, r)
        rows_x = h_all[:, l2g].reshape(-1, d.hidden)
        rows_dy = dy[:, l2g].reshape(-1, d.hidden)
        share = bwd.rank_mlp_backward(rows_x, rows_dy, inp, dataclasses.replace(d, rank=r))
        full = bwd.mlp_backward(rows_x, wg, wu, wd, rows_dy)
        np.testing.assert_allclose(share["dx"], full["dx"], rtol=1e-11, atol=1e-12)
        for k in tot:
            tot[k] = tot[k] + share[k]
    want = bwd.mlp_backward(h_all.reshape(-1, d.hidden), wg, wu, wd, dy.reshape(-1, d.hidden))
    for k in tot:
        np.testing.assert_allclose(tot[k], want[k], rtol=1e-11, atol=1e-12, err_msg=k)


def test_silu_grad_closed_forms():
    z = np.array([0.0, 1.0, -2.0, 40.0, -40.0])
    s = 1 / (1 + np.exp(-z))
    np.testing.assert_allclose(bwd.silu_grad(z), s + z * s * (1 - s), rtol=1e-14)
    assert bwd.silu_grad(np.array([0.0]))[0] == 0.5
    zt = torch.tensor(z, requires_grad=True)
    torch.nn.functional.silu(zt).sum().backward()
    np.testing.assert_allclose(bwd.silu_grad(z), zt.grad.numpy(), rtol=1e-14, atol=1e-300)


@pytest.mark.parametrize("shape", TINY)
@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
def test_rank_attention_shares_sum_to_the_unsharded_gradients(shape, partition):
    # every rank's share of the attention backward: its input gradient rows
    # equal the unsharded dx - dh; its K/V contributions summed over ranks
    # are the unsharded ones; its weight-gradient shares sum to dW_Q/K/V/O
    d, inp, dy = _setup(shape, seed=35)
    d = dataclasses.replace(d, partition=partition)
    full = bwd.layer_backward(inp, d, dy)
    B, S, D = d.batch, d.seq, d.degree
    hq_s, hkv_s, dh = d.n_q_heads // D, d.n_kv_heads // D, d.head_dim
    tot_o = 0.0
    tot_qkv = 0.0
    contrib = 0.0
    for r in range(D):
        dr = dataclasses.replace(d, rank=r)
        sh = bwd.rank_attention_backward(inp, dr, full["dh"])
        rows = orc.local_to_global(S, D, r, partition)
        np.testing.assert_allclose(sh["dx_attn"], (full["dx"] - full["dh"])[:, rows], rtol=1e-10, atol=1e-11)
        tot_o = tot_o + sh["dw_o"]
        tot_qkv = tot_qkv + sh["dw_qkv"]
        contrib = contrib + sh["dkv_contrib"]
    np.testing.assert_allclose(tot_o, full["dw_o"], rtol=1e-10, atol=1e-11)
    # packed per-shard rows -> unsharded dW_q, dW_k, dW_v
    for j in range(D):
        ql = slice(j * hq_s * dh, (j + 1) * hq_s * dh)
        kl = slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        np.testing.assert_allclose(tot_qkv[j, :hq_s * dh], full["dw_q"][ql], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(tot_qkv[j, hq_s * dh:(hq_s + hkv_s) * dh], full["dw_k"][kl], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(tot_qkv[j, (hq_s + hkv_s) * dh:], full["dw_v"][kl], rtol=1e-10, atol=1e-11)
    # the summed contributions are the whole sequence's dK, dV (x^T of them = dW_K, dW_V)
    x = orc.bf16_bits_to_f64(inp["x"])
    for j in range(D):
        kl = slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        np.testing.assert_allclose(np.einsum("bsk,bsh->kh", contrib[j, 0], x), full["dw_k"][kl], rtol=1e-10,
                                   atol=1e-11)
        np.testing.assert_allclose(np.einsum("bsk,bsh->kh", contrib[j, 1], x), full["dw_v"][kl], rtol=1e-10,
                                   atol=1e-11)
