"""Pins for the CPU oracle against things other than itself.

Each check here fixes a part of ``oracle/tsp_oracle.py`` by a hand-written
fixture, a closed form, an independent brute-force loop, or an independent
library routine (PyTorch's float64 CPU attention / silu), so that a dropped
term, a wrong sign or index, or a transposed operand in the oracle fails one of
them.  CPU only.
"""
import itertools
import dataclasses
import math
import os

import numpy as np
import pytest
import torch

import synth
from oracle import tsp_oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------- #
# bfloat16 decoding and rounding (input plumbing)
# --------------------------------------------------------------------------- #
def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x3E80, 0x0000, 0x8000, 0x4049, 0x3C23], dtype=np.uint16)
    want = [1.0, -2.0, 0.25, 0.0, -0.0, 3.140625, 0.009948730468750]
    got = orc.bf16_bits_to_f64(bits)
    assert got.tolist() == want


def test_rne_rounding_of_generator():
    # 1 + 2^-8 is a tie between 1.0 and 1 + 2^-7: ties go to the even mantissa (1.0);
    # 1 + 3*2^-9 rounds up; 1 + 3*2^-8 is a tie going up to the even 1 + 2^-6.
    a = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -9, 1 + 3 * 2.0 ** -8, -1 - 2.0 ** -8], np.float32)
    bits = synth.f32_to_bf16_bits(a)
    assert orc.bf16_bits_to_f64(bits).tolist() == [1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6, -1.0]


def test_generator_row_prefix_is_stable():
    d = synth.Dims(1, 64, 2, 0, 32, 2, 2, 16, 64)
    full = synth.make_inputs(d, 0.02, 7)
    part = synth.make_inputs(d, 0.02, 7, x_rows=20)
    assert np.array_equal(full["x"][:, :20], part["x"])
    for k in ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d"):
        assert np.array_equal(full[k], part[k])


# --------------------------------------------------------------------------- #
# P1: zigzag maps
# --------------------------------------------------------------------------- #
def _golden_zigzag(name="zigzag_maps.txt"):
    l2g, g2s = {}, {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            head, vals = line.split(":")
            S, D, r = head.split()
            vals = [int(v) for v in vals.split()]
            if r == "gs":
                g2s[(int(S), int(D))] = vals
            else:
                l2g[(int(S), int(D), int(r))] = vals
    return l2g, g2s


def test_zigzag_golden():
    l2g, g2s = _golden_zigzag()
    assert len(l2g) >= 8 and len(g2s) >= 2
    for (S, D, r), want in l2g.items():
        assert orc.local_to_global(S, D, r).tolist() == want
    for (S, D), want in g2s.items():
        assert orc.global_to_slot(S, D).tolist() == want


@pytest.mark.parametrize("S,D", [(4, 1), (8, 2), (48, 3), (64, 4), (96, 8), (256, 8), (8192, 8)])
def test_zigzag_is_permutation_and_inverse(S, D):
    T = S // D
    allg = np.concatenate([orc.local_to_global(S, D, r) for r in range(D)])
    assert sorted(allg.tolist()) == list(range(S))
    slot = orc.global_to_slot(S, D)
    for r in range(D):
        g = orc.local_to_global(S, D, r)
        assert slot[g].tolist() == list(range(r * T, (r + 1) * T))
    if D == 1:
        assert orc.local_to_global(S, 1, 0).tolist() == list(range(S))


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_zigzag_equal_causal_pairs(name):
    # Each rank's causal pair count is c(2Dc+1) = S(S+1)/(2D): the balance the
    # zigzag partition is chosen for.  Brute force over every rank.
    d = synth.WORKLOADS[name].dims
    S, D = d.seq, d.degree
    c = S // (2 * D)
    want = c * (2 * D * c + 1)
    assert want * 2 * D == S * (S + 1)
    ranks = range(D) if S <= 16384 else [0, D - 1, d.rank]
    for r in ranks:
        assert orc.causal_pairs(S, D, r) == want


# Striped partition (the alternative to zigzag): golden maps written by hand,
# permutation / inverse, and a closed form for the causal pairs, which are no
# longer equal over ranks: rank r's row t sits at tD + r, so it has
# D T (T - 1) / 2 + T (r + 1) pairs.
def test_striped_golden():
    l2g, g2s = _golden_zigzag("striped_maps.txt")
    assert len(l2g) >= 6 and len(g2s) >= 2
    for (S, D, r), want in l2g.items():
        assert orc.local_to_global(S, D, r, orc.STRIPED).tolist() == want
    for (S, D), want in g2s.items():
        assert orc.global_to_slot(S, D, orc.STRIPED).tolist() == want


@pytest.mark.parametrize("S,D", [(4, 1), (8, 2), (48, 3), (96, 8), (8192, 8)])
def test_striped_is_permutation_and_inverse(S, D):
    T = S // D
    allg = np.concatenate([orc.local_to_global(S, D, r, orc.STRIPED) for r in range(D)])
    assert sorted(allg.tolist()) == list(range(S))
    slot = orc.global_to_slot(S, D, orc.STRIPED)
    for r in range(D):
        g = orc.local_to_global(S, D, r, orc.STRIPED)
        assert slot[g].tolist() == list(range(r * T, (r + 1) * T))
        assert orc.causal_pairs(S, D, r, orc.STRIPED) == D * T * (T - 1) // 2 + T * (r + 1)
    # every rank's pairs sum to the whole causal triangle, as for zigzag
    assert sum(orc.causal_pairs(S, D, r, orc.STRIPED) for r in range(D)) == S * (S + 1) // 2
    if D == 1:
        assert orc.local_to_global(S, 1, 0, orc.STRIPED).tolist() == list(range(S))


def test_zigzag_rejects_bad_dims():
    with pytest.raises(ValueError):
        orc.local_to_global(10, 3, 0)
    with pytest.raises(ValueError):
        orc.local_to_global(16, 2, 2)
    with pytest.raises(ValueError):
        orc.local_to_global(16, 2, 0, partition=2)


# --------------------------------------------------------------------------- #
# Attention: brute force, closed forms, and an independent library routine
# --------------------------------------------------------------------------- #
def _bruteforce_attention(q, k, v, pos, scale):
    n, dh = q.shape
    out = [[0.0] * v.shape[1] for _ in range(n)]
    for i in range(n):
        logits = []
        for j in range(int(pos[i]) + 1):
            logits.append(sum(q[i][d] * k[j][d] for d in range(dh)) * scale)
        mx = max(logits)
        w = [math.exp(t - mx) for t in logits]
        tot = sum(w)
        for e in range(v.shape[1]):
            out[i][e] = sum(w[j] * v[j][e] for j in range(len(w))) / tot
    return np.array(out)


def test_attention_matches_bruteforce_tiny():
    rng = np.random.default_rng(11)
    nk, dh, dv = 13, 5, 3  # dv != dh catches a transposed V
    k = rng.standard_normal((nk, dh))
    v = rng.standard_normal((nk, dv))
    pos = np.array([0, 3, 7, 12, 2])
    q = rng.standard_normal((len(pos), dh)) * 2.0
    got = orc.causal_attention(q, k, v, pos, block=2)
    want = _bruteforce_attention(q, k, v, pos, 1.0 / math.sqrt(dh))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("hq,hkv", [(4, 4), (4, 2), (8, 1)])
def test_attention_matches_torch_sdpa(hq, hkv):
    rng = np.random.default_rng(12)
    S, dh = 40, 16
    q = rng.standard_normal((hq, S, dh))
    k = rng.standard_normal((hkv, S, dh))
    v = rng.standard_normal((hkv, S, dh))
    kt = torch.from_numpy(k).repeat_interleave(hq // hkv, dim=0)
    vt = torch.from_numpy(v).repeat_interleave(hq // hkv, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], kt[None], vt[None], is_causal=True)[0].numpy()
    for i in range(hq):
        got = orc.causal_attention(q[i], k[i // (hq // hkv)], v[i // (hq // hkv)], np.arange(S))
        np.testing.assert_allclose(got, want[i], rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(13)
    S, dh = 24, 8
    k = rng.standard_normal((S, dh))
    v = rng.standard_normal((S, dh))
    pos = np.arange(S)
    # Q = 0: uniform weights over the causal prefix -> prefix mean of V
    o = orc.causal_attention(np.zeros((S, dh)), k, v, pos)
    want = np.cumsum(v, axis=0) / np.arange(1, S + 1)[:, None]
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)
    # constant V: every output equals that row
    vc = np.tile(rng.standard_normal(dh), (S, 1))
    o = orc.causal_attention(rng.standard_normal((S, dh)), k, vc, pos)
    np.testing.assert_allclose(o, vc, rtol=1e-13, atol=1e-13)
    # first position sees only key 0
    o = orc.causal_attention(rng.standard_normal((1, dh)), k, v, np.array([0]))
    np.testing.assert_allclose(o[0], v[0], rtol=0, atol=0)
    # one key with a huge logit dominates
    kk = np.zeros((S, dh)); kk[5, 0] = 1.0
    qq = np.zeros((1, dh)); qq[0, 0] = 1e4
    o = orc.causal_attention(qq, kk, v, np.array([S - 1]))
    np.testing.assert_allclose(o[0], v[5], rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- #
# silu / SwiGLU
# --------------------------------------------------------------------------- #
def test_silu_known_values_and_library():
    z = np.array([0.0, 1.0, -1.0, 2.0, 50.0, -50.0, 800.0, -800.0])
    s = orc.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-15     # 1/(1+e^-1)
    assert abs(s[2] + 0.2689414213699951) < 1e-15     # -1/(1+e)
    assert abs(s[3] - 1.7615941559557646) < 1e-15     # 2/(1+e^-2)
    assert s[6] == 800.0
    assert abs(s[7]) < 1e-300
    zz = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(orc.silu(zz), torch.nn.functional.silu(torch.from_numpy(zz)).numpy(),
                               rtol=1e-14, atol=1e-300)


def test_swiglu_matches_bruteforce():
    rng = np.random.default_rng(14)
    n, h, F = 3, 5, 7
    x = rng.standard_normal((n, h))
    wg = rng.standard_normal((F, h))
    wu = rng.standard_normal((F, h))
    wd = rng.standard_normal((h, F))
    got = orc.swiglu_mlp(x, wg, wu, wd)
    want = np.zeros((n, h))
    for i in range(n):
        a = []
        for f in range(F):
            g = sum(x[i][e] * wg[f][e] for e in range(h))
            u = sum(x[i][e] * wu[f][e] for e in range(h))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for e in range(h):
            want[i][e] = sum(a[f] * wd[e][f] for f in range(F))
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


# --------------------------------------------------------------------------- #
# Whole layer: brute force on a tiny shape, and an independent torch float64
# implementation of the unsharded layer on the tiny workload
# --------------------------------------------------------------------------- #
def _bruteforce_layer(inputs, d, r):
    """Pure-Python loops: h = x + Attn(x), y = h + SwiGLU(h), rank r's rows."""
    dec = orc.bf16_bits_to_f64
    X = dec(inputs["x"])
    Wq, Wk, Wv, Wo = (dec(inputs[n]) for n in ("w_q", "w_k", "w_v", "w_o"))
    Wg, Wu, Wd = (dec(inputs[n]) for n in ("w_g", "w_u", "w_d"))
    S, D, h, Hq, Hkv, dh, F = d.seq, d.degree, d.hidden, d.n_q_heads, d.n_kv_heads, d.head_dim, d.ffn
    c = S // (2 * D)
    rows = list(range(r * c, (r + 1) * c)) + list(range((2 * D - 1 - r) * c, (2 * D - r) * c))
    out = np.zeros((d.batch, len(rows), h))
    lin = lambda x, W: [sum(x[e] * W[o][e] for e in range(len(x))) for o in range(len(W))]
    for b in range(d.batch):
        K = [lin(X[b][s], Wk) for s in range(S)]
        V = [lin(X[b][s], Wv) for s in range(S)]
        for t, g in enumerate(rows):
            Q = lin(X[b][g], Wq)
            O = [0.0] * (Hq * dh)
            for i in range(Hq):
                kv = i * Hkv // Hq
                lg = [sum(Q[i * dh + e] * K[s][kv * dh + e] for e in range(dh)) / math.sqrt(dh)
                      for s in range(g + 1)]
                m = max(lg)
                w = [math.exp(a - m) for a in lg]
                z = sum(w)
                for e in range(dh):
                    O[i * dh + e] = sum(w[s] * V[s][kv * dh + e] for s in range(g + 1)) / z
            hh = [X[b][g][e] + v for e, v in enumerate(lin(O, Wo))]
            gt, up = lin(hh, Wg), lin(hh, Wu)
            a = [gt[f] / (1 + math.exp(-gt[f])) * up[f] for f in range(F)]
            out[b, t] = [hh[e] + v for e, v in enumerate(lin(a, Wd))]
    return out


@pytest.mark.parametrize("r", [0, 1])
def test_layer_matches_bruteforce_tiny_gqa(r):
    # non-square everywhere: h=6, Hq*dh=8, Hkv*dh=4, F=10, B=2
    d, inp = synth.make_custom(2, 8, 2, r, 6, 4, 2, 2, 10, sigma=0.4, seed=21)
    got = orc.layer_rank_rows(inp, d)["y"]
    want = _bruteforce_layer(inp, d, r)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_layer_matches_torch_float64_tiny_workload():
    w = synth.WORKLOADS["tiny_d2"]
    d = w.dims
    inp = synth.make_inputs(d, w.sigma, w.seed)
    got = orc.layer_rank_rows(inp, d)
    # Independent implementation with torch float64 CPU ops on the whole sequence.
    dec = lambda n: torch.from_numpy(orc.bf16_bits_to_f64(inp[n]))
    X = dec("x")[0]
    q = (X @ dec("w_q").T).view(d.seq, d.n_q_heads, d.head_dim).transpose(0, 1)
    k = (X @ dec("w_k").T).view(d.seq, d.n_kv_heads, d.head_dim).transpose(0, 1)
    v = (X @ dec("w_v").T).view(d.seq, d.n_kv_heads, d.head_dim).transpose(0, 1)
    rep = d.n_q_heads // d.n_kv_heads
    o = torch.nn.functional.scaled_dot_product_attention(
        q[None], k.repeat_interleave(rep, 0)[None], v.repeat_interleave(rep, 0)[None], is_causal=True)[0]
    o = o.transpose(0, 1).reshape(d.seq, -1)
    H = X + o @ dec("w_o").T
    Y = H + (torch.nn.functional.silu(H @ dec("w_g").T) * (H @ dec("w_u").T)) @ dec("w_d").T
    # rank 0 of D=2 holds chunks 0 and 3 of 64 rows (golden-style literal slice)
    rows = list(range(0, 64)) + list(range(192, 256))
    np.testing.assert_allclose(got["y"][0], Y[rows].numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(got["h"][0], H[rows].numpy(), rtol=1e-11, atol=1e-11)


# --------------------------------------------------------------------------- #
# P2 / P3 / P6 / P7: the TSP schedule reproduces the unsharded layer
# --------------------------------------------------------------------------- #
def test_mlp_shard_sum_identity():
    rng = np.random.default_rng(15)
    n, h, F, D = 9, 16, 24, 4
    x = rng.standard_normal((n, h))
    wg, wu = rng.standard_normal((F, h)), rng.standard_normal((F, h))
    wd = rng.standard_normal((h, F))
    fs = F // D
    parts = sum(orc.swiglu_mlp(x, wg[j * fs:(j + 1) * fs], wu[j * fs:(j + 1) * fs], wd[:, j * fs:(j + 1) * fs])
                for j in range(D))
    np.testing.assert_allclose(parts, orc.swiglu_mlp(x, wg, wu, wd), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("shape", [
    (1, 32, 2, 0, 16, 2, 2, 8, 24),    # MHA, D=2
    (2, 48, 3, 0, 12, 6, 3, 4, 18),    # GQA 2:1, D=3, B=2
    (1, 64, 4, 0, 16, 8, 4, 4, 32),    # GQA, D=4
])
@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
def test_tsp_schedule_equals_unsharded_layer(shape, partition):
    d0, inp = synth.make_custom(*shape, sigma=0.3, seed=31)
    d0 = dataclasses.replace(d0, partition=partition)
    ys = orc.tsp_schedule(inp, d0)
    for r in range(d0.degree):
        d = dataclasses.replace(d0, rank=r)
        ref = orc.layer_rank_rows(inp, d)["y"]
        np.testing.assert_allclose(ys[r], ref, rtol=1e-12, atol=1e-12)
        # the rank's rows are the unsharded layer's rows at its positions:
        # slicing the full-sequence result by the partition map gives them too
        if r == 0:
            full = orc.layer_rank_rows(inp, dataclasses.replace(d0, degree=1, rank=0))["y"]
            np.testing.assert_allclose(ys[r], full[:, orc.local_to_global(d0.seq, d0.degree, 0, partition)],
                                       rtol=1e-12, atol=1e-12)


def test_rows_subset_equals_full_slice():
    w = synth.WORKLOADS["tiny_d2"]
    inp = synth.make_inputs(w.dims, w.sigma, w.seed)
    full = orc.layer_rank_rows(inp, w.dims)
    rows = np.array([0, 1, 63, 64, 65, 127])
    part = orc.layer_rank_rows(inp, w.dims, rows=rows)
    for key in ("y", "h", "attn", "mlp"):
        np.testing.assert_allclose(part[key], full[key][:, rows], rtol=1e-14, atol=1e-14)


# --------------------------------------------------------------------------- #
# Work accounting closed forms
# --------------------------------------------------------------------------- #
def test_algorithmic_flops_llama7b_8k():
    d = synth.WORKLOADS["llama7b_s8k_d8"].dims
    f = orc.algorithmic_flops(d)
    M, h = 1024, 4096
    assert f["qkv"] == 2 * M * 3 * 4096 * h
    assert f["o"] == 2 * M * 4096 * h
    assert f["attn"] == 4 * 128 * 32 * (8192 * 8193 // 16)
    assert f["mlp"] == 2 * M * 3 * 11008 * h
    assert abs(f["total"] / 1e9 - 483.2) < 0.05


# --------------------------------------------------------------------------- #
# qkv_rows and mlp_block, the per-kernel references of the GPU tests
# --------------------------------------------------------------------------- #
def _tiny_gqa_inputs(seed=21, sigma=0.5):
    # non-square everywhere: Hq != Hkv, dh != h, F != h, B = 2, D = 2
    d = synth.Dims(2, 8, 2, 0, 8, 4, 2, 4, 12)
    return d, synth.make_inputs(d, sigma, seed)


@pytest.mark.parametrize("rank", [0, 1])
def test_qkv_rows_matches_bruteforce_every_source_rank(rank):
    """X W^T of every local row of rank `rank`, as a triple loop over the
    positions the zigzag rule gives that rank written out by hand (chunks r
    and 2D-1-r of c = 2 positions: rank 0 holds 0, 1, 6, 7; rank 1 holds 2, 3,
    4, 5), so a wrong source rank, row order or weight fails."""
    d, inp = _tiny_gqa_inputs()
    d = dataclasses.replace(d, rank=rank)
    positions = {0: [0, 1, 6, 7], 1: [2, 3, 4, 5]}[rank]
    x = orc.bf16_bits_to_f64(inp["x"])
    for b in range(d.batch):
        got = orc.qkv_rows(inp, d, b, np.arange(4))
        # also through the rank argument while dims says the other rank
        other = dataclasses.replace(d, rank=1 - rank)
        got2 = orc.qkv_rows(inp, other, b, np.arange(4), rank=rank)
        for name in ("q", "k", "v"):
            w = orc.bf16_bits_to_f64(inp["w_" + name])
            want = np.zeros((4, w.shape[0]))
            for t, g in enumerate(positions):
                for o in range(w.shape[0]):
                    acc = 0.0
                    for k in range(d.hidden):
                        acc += x[b, g, k] * w[o, k]
                    want[t, o] = acc
            np.testing.assert_allclose(got[name], want, rtol=1e-13, atol=1e-14)
            np.testing.assert_array_equal(got2[name], got[name])
    # the three projections are distinct (a swapped weight would show)
    assert not np.allclose(got["k"], got["v"])


def test_mlp_block_matches_bruteforce_and_torch():
    """x + (silu(x Wg^T) * (x Wu^T)) Wd^T row by row in plain loops, and
    through PyTorch's float64 silu and matmul; gate and up swapped, or the
    residual dropped, fail (checked below)."""
    d, inp = _tiny_gqa_inputs(seed=22)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, d.hidden))
    wg, wu, wd = (orc.bf16_bits_to_f64(inp[n]) for n in ("w_g", "w_u", "w_d"))
    got = orc.mlp_block(inp, x)
    want = np.zeros_like(x)
    for i in range(x.shape[0]):
        a = []
        for f in range(d.ffn):
            g = sum(x[i, k] * wg[f, k] for k in range(d.hidden))
            u = sum(x[i, k] * wu[f, k] for k in range(d.hidden))
            a.append(g / (1.0 + math.exp(-g)) * u)
        for o in range(d.hidden):
            want[i, o] = x[i, o] + sum(a[f] * wd[o, f] for f in range(d.ffn))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    xt = torch.from_numpy(x)
    ref = xt + (torch.nn.functional.silu(xt @ torch.from_numpy(wg).T) * (xt @ torch.from_numpy(wu).T)) \
        @ torch.from_numpy(wd).T
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-13)
    # the pins are sharp enough to see the plausible slips
    swapped = x + (orc.silu(x @ wu.T) * (x @ wg.T)) @ wd.T
    assert np.abs(swapped - want).max() > 1e-3
    assert np.abs((got - x) - want).max() > 1e-1
