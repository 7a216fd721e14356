"""The f16 storage-rounding model (``oracle/rounding_model.py``): pinned to the
oracle and to IEEE binary16, then used to show where each workload's error
floor lies against the tolerance (max-abs 2e-2, rel-Frobenius 5e-3).  CPU only."""
import functools

import numpy as np
import pytest

import synth
from oracle import rounding_model as rm
from oracle import tsp_oracle as orc
from gpu_util import sample_rows


def test_f16_rounding_known_values():
    # binary16 has a 10-bit fraction: spacing 2^-10 in [1, 2), ties to even
    ulp = 2.0 ** -10
    vals = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, 1 + ulp / 2 + 2 ** -30, 65504.0, 2.0 ** -24, 2.0 ** -26, -3.0])
    want = np.array([1.0, 1 + 2 * ulp, 1 + ulp, 65504.0, 2.0 ** -24, 0.0, -3.0])
    assert np.array_equal(rm.f16(vals), want)


def test_without_rounding_points_it_is_the_oracle():
    wl = synth.WORKLOADS["tiny_d2"]
    d = wl.dims
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    rows = np.arange(d.seq // d.degree)
    ref = orc.rank_rows_forward(inp, d, 0, rows)["y"]
    got = rm.rank_rows_rounded(inp, d, 0, rows, points=())
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        rm.rank_rows_rounded(inp, d, 0, rows, points=("bf16",))


def test_each_rounding_point_changes_the_result():
    # every point is wired in: enabling it alone moves y, by an amount of the
    # order of f16 spacing times the activations
    wl = synth.WORKLOADS["tiny_d2"]
    d = wl.dims
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    rows = np.arange(d.seq // d.degree)
    ref = rm.rank_rows_rounded(inp, d, 0, rows, points=())
    scale = np.abs(ref).max()
    for p in rm.POINTS:
        err = np.abs(rm.rank_rows_rounded(inp, d, 0, rows, points=(p,)) - ref).max()
        assert 0 < err < 64 * 2.0 ** -11 * scale, p


@functools.lru_cache(maxsize=None)
def _setup(name):
    wl = synth.WORKLOADS[name]
    d = wl.dims
    T, c = d.seq // d.degree, d.seq // (2 * d.degree)
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    rows = sample_rows(T, c)
    g = orc.local_to_global(d.seq, d.degree, d.rank)[rows]
    kv = orc.project_kv(inp, d, 0, int(g.max()) + 1)
    w = {n: orc.bf16_bits_to_f64(inp[n]) for n in ("w_q", "w_o", "w_g", "w_u", "w_d")}
    ref = orc.rank_rows_forward(inp, d, 0, rows, kv=kv, weights=w)["y"]
    return d, inp, rows, kv, w, ref


def _floor(name, points=rm.POINTS):
    d, inp, rows, kv, w, ref = _setup(name)
    y = rm.rank_rows_rounded(inp, d, 0, rows, points=points, kv=kv, weights=w)
    return np.abs(y - ref).max(), np.linalg.norm(y - ref) / np.linalg.norm(ref)


def test_llama7b_floor_is_inside_the_tolerance():
    max_abs, rel = _floor("llama7b_s8k_d8")
    assert max_abs < 2e-2 and rel < 5e-3


def test_wide70b_floor_exceeds_the_max_abs_bar():
    # the 70B-like layer (hidden 8192, |y| ~ 50 at the first tokens) cannot
    # meet max-abs 2e-2 with f16 storage at all; rel-Frobenius stays ~10x inside
    max_abs, rel = _floor("wide70b_s32k_d8")
    assert 2e-2 < max_abs < 3e-2
    assert rel < 1e-3


def test_wide70b_cheap_widening_does_not_reach_the_bar():
    # The one widening that costs under 7% of the layer's matrix-core work is
    # the attention output O kept wide into the output projection (an f16
    # hi + lo pair doubles that 550-GFLOP GEMM: +6%).  It leaves the floor
    # above 2e-2; the pairs that get under it (Q/K/V with O, or the MLP's
    # two inputs h16 and act) double attention or MLP products (+36%..+63%).
    max_abs, _ = _floor("wide70b_s32k_d8", points=tuple(p for p in rm.POINTS if p != "o"))
    assert max_abs > 2e-2
    max_abs, _ = _floor("wide70b_s32k_d8", points=("qkv", "p", "o"))   # h16 and act wide
    assert max_abs < 2e-2


# --------------------------------------------------------------------------- #
# Backward of the gated MLP: bfloat16 storage points
# --------------------------------------------------------------------------- #
def test_bf16_rounding_known_values():
    # bfloat16 keeps 7 fraction bits: spacing 2^-7 in [1, 2), ties to even;
    # float32's range (no overflow at 1e38, normals down to 2^-126)
    ulp = 2.0 ** -7
    vals = np.array([1 + ulp / 2, 1 + 3 * ulp / 2, 1 + ulp / 2 + 2 ** -20, 3e38, 2.0 ** -126, -1.0])
    # 3e38 = 1.7632 x 2^127: the nearest 7-bit fraction is 98/128
    want = np.array([1.0, 1 + 2 * ulp, 1 + ulp, (1 + 98 / 128) * 2.0 ** 127, 2.0 ** -126, -1.0])
    assert np.array_equal(rm.bf16(vals), want)


def _mlp_case(seed=41, n=24, h=32, F=48):
    rng = np.random.default_rng(seed)
    x = rm.bf16(rng.standard_normal((n, h)))
    dy = rng.standard_normal((n, h))
    wg, wu = rm.bf16(0.1 * rng.standard_normal((F, h))), rm.bf16(0.1 * rng.standard_normal((F, h)))
    wd = rm.bf16(0.1 * rng.standard_normal((h, F)))
    return x, wg, wu, wd, dy


def test_backward_model_without_rounding_is_the_oracle():
    from oracle import tsp_backward as bwd
    x, wg, wu, wd, dy = _mlp_case()
    ref = bwd.mlp_backward(x, wg, wu, wd, dy)
    got = rm.mlp_backward_rounded(x, wg, wu, wd, dy, points=())
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        np.testing.assert_allclose(got[k], ref[k], rtol=1e-12, atol=1e-13, err_msg=k)
    with pytest.raises(ValueError):
        rm.mlp_backward_rounded(x, wg, wu, wd, dy, points=("o",))


def test_backward_bf16_floor_sits_inside_the_relative_bars():
    # every storage point rounded to bf16 leaves each gradient about 2.4e-3
    # (relative Frobenius) and 3e-3 (max-abs over the largest element) from
    # the float64 result: the GPU tests hold the backward to 5e-3 and 2e-2
    from oracle import tsp_backward as bwd
    x, wg, wu, wd, dy = _mlp_case(n=256, h=128, F=384)
    ref = bwd.mlp_backward(x, wg, wu, wd, dy)
    got = rm.mlp_backward_rounded(x, wg, wu, wd, dy)
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        diff = got[k] - ref[k]
        rel = np.linalg.norm(diff) / np.linalg.norm(ref[k])
        ma = np.abs(diff).max() / np.abs(ref[k]).max()
        assert 1e-3 < rel < 3.5e-3 and ma < 1e-2, (k, rel, ma)
