"""GPU parity of the MLP-ring backward (tsp_mlp_ring_bwd, through the C ABI)
against the float64 backward oracle.

The reference is the oracle's share of rank r (``rank_mlp_backward``): the
input gradient of the rank's tokens and their contribution to every shard's
weight gradients.  Bars, relative to each output: max-abs over the largest
reference element <= 2e-2 and relative Frobenius <= 5e-3 (the bfloat16
storage floor of the gradients sits at 3e-3 and 2.4e-3:
tests/test_rounding_floor.py).
"""
import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_amd import binding as B
from folded_tensor_sequence_amd.harness import pack_weights
from oracle import tsp_backward as bwd
from oracle import tsp_oracle as orc

from gpu_util import MAX_ABS, REL_FROB, SWEEP, dims_of, errors, inputs_for, tuning

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _shape(name):
    if name in synth.WORKLOADS:
        w = synth.WORKLOADS[name]
        return w.dims, w.sigma, w.seed
    return dims_of(SWEEP[name]), 0.02, 101


def _check(name, got, ref):
    ma, rf = errors(got, ref)
    ma_rel = ma / float(np.abs(ref).max())
    print(f"  {name}: max_abs/max={ma_rel:.3e} rel_frob={rf:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert ma_rel <= MAX_ABS and rf <= REL_FROB, (name, ma_rel, rf)


def _run(d, inp, xdt, with_residual=True, seed=7):
    """Runs tsp_mlp_ring_bwd on rank d.rank's rows; returns GPU outputs and the
    oracle's."""
    T = d.seq // d.degree
    w = {k: v.cuda() for k, v in pack_weights(inp, d).items()}
    l2g = orc.local_to_global(d.seq, d.degree, d.rank, getattr(d, "partition", 0))
    bits = np.ascontiguousarray(inp["x"][:, l2g])
    x64 = orc.bf16_bits_to_f64(bits)
    if xdt == "bf16":
        xt, xval, kw = torch.from_numpy(bits.view(np.int16)).cuda(), x64, {"x_dtype": B.TSP_BF16}
    elif xdt == "f16":
        h16 = (x64 * 1.25).astype(np.float16)
        xt, xval, kw = torch.from_numpy(h16).cuda(), h16.astype(np.float64), {}
    else:
        f32 = (x64 * 1.25).astype(np.float32)
        xt, xval, kw = torch.from_numpy(f32).cuda(), f32.astype(np.float64), {}
    dy = np.ascontiguousarray(synth.make_grad(d, seed)[:, l2g])
    dyt = torch.from_numpy(dy).cuda()
    dx = torch.empty_like(dyt)
    F, h, D = d.ffn, d.hidden, d.degree
    dwg = torch.empty((F, h), dtype=torch.float32, device="cuda")
    dwu = torch.empty_like(dwg)
    dwd = torch.empty((D, h, F // D), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_MLP_BWD), dtype=torch.uint8, device="cuda")
    B.tsp_mlp_ring_bwd(d, xt, dyt, w["w_gate"], w["w_up"], w["w_down"], dx, dwg, dwu, dwd, ws,
                       dx_residual=dyt if with_residual else None, **kw)
    torch.cuda.synchronize()
    ref = bwd.rank_mlp_backward(xval.reshape(-1, h), dy.astype(np.float64).reshape(-1, h), inp, d)
    ref_dx = ref["dx"].reshape(d.batch, T, h) + (dy if with_residual else 0.0)
    ref_dwd = np.stack([ref["dw_d"][:, j * (F // D):(j + 1) * (F // D)] for j in range(D)])
    gpu = {"dx": dx.cpu().numpy(), "dw_g": dwg.cpu().numpy(), "dw_u": dwu.cpu().numpy(),
           "dw_d": dwd.cpu().numpy()}
    return gpu, {"dx": ref_dx, "dw_g": ref["dw_g"], "dw_u": ref["dw_u"], "dw_d": ref_dwd}, \
        (xt, dyt, w, ws, kw, dx, dwg, dwu, dwd)


# Shapes: the tiny layer; MLP shards of 176 and 96 columns (not multiples of
# 64: ragged K segments of the input gradient and ragged transposes); B = 2;
# D = 1; 48 rows (token axis padded to 64); a wider hidden size.
SMALL = ["tiny_d2", "mha_d2_r1", "ffn_tail_d4_r3", "gqa8_b2_c96", "d1", "c24_generic_reorder", "wide_tiles_dh128"]


@pytest.mark.parametrize("name", SMALL)
@pytest.mark.parametrize("xdt", ["bf16", "f16", "f32"])
def test_mlp_ring_bwd(name, xdt):
    d, sigma, seed = _shape(name)
    _case(f"mlp_ring_bwd {name} x={xdt}")
    inp = inputs_for(d.astuple(), sigma, seed)
    gpu, ref, _ = _run(d, inp, xdt)
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        _check(k, gpu[k], ref[k])


@pytest.mark.parametrize("name", ["tiny_d2", "ffn_tail_d4_r3"])
def test_mlp_ring_bwd_without_residual_in_place_and_deterministic(name):
    d, sigma, seed = _shape(name)
    _case(f"mlp_ring_bwd {name} residual=NULL, in place, twice")
    inp = inputs_for(d.astuple(), sigma, seed)
    gpu, ref, (xt, dyt, w, ws, kw, dx, dwg, dwu, dwd) = _run(d, inp, "bf16", with_residual=False)
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        _check(k, gpu[k], ref[k])
    # in place: dx written over dy (dy consumed first), with dy as the residual
    keep = {k: v.clone() for k, v in (("dwg", dwg), ("dwu", dwu), ("dwd", dwd))}
    dy_in = dyt.clone()
    B.tsp_mlp_ring_bwd(d, xt, dy_in, w["w_gate"], w["w_up"], w["w_down"], dy_in, dwg, dwu, dwd, ws,
                       dx_residual=dy_in, **kw)
    torch.cuda.synchronize()
    B.tsp_mlp_ring_bwd(d, xt, dyt, w["w_gate"], w["w_up"], w["w_down"], dx, dwg, dwu, dwd, ws,
                       dx_residual=dyt, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dy_in, dx)
    # the weight gradients do not depend on the residual and repeat bit for bit
    for k, v in (("dwg", dwg), ("dwu", dwu), ("dwd", dwd)):
        assert torch.equal(v, keep[k]), k


# dA = dy W_down and dx = sum dG_j W_gate,j + dU_j W_up,j read the weights as
# stored (K-major products); TSP_TUNE_BWD_WEIGHTS = 1 multiplies by
# transposed copies instead.  Both sum every product in the same K order, so
# the outputs agree bit for bit (the default path is the one held to the
# oracle above).  ffn_tail_d4_r3 (F/D = 176) takes the copies for dx either
# way.
@pytest.mark.parametrize("name", ["tiny_d2", "gqa8_b2_c96", "ffn_tail_d4_r3", "wide_tiles_dh128"])
def test_mlp_ring_bwd_weight_copies_match_kmajor(name):
    d, sigma, seed = _shape(name)
    _case(f"mlp_ring_bwd {name} weights as stored vs transposed copies")
    inp = inputs_for(d.astuple(), sigma, seed)
    gpu, _, _ = _run(d, inp, "bf16")
    with tuning(bwd_weights=1):
        gpu_t, ref, _ = _run(d, inp, "bf16")
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        _check(k, gpu_t[k], ref[k])
        assert np.array_equal(gpu[k], gpu_t[k]), k


# Rank 5 of D = 8 (the ring starts at shard 5) and the striped partition.
def test_mlp_ring_bwd_middle_rank_striped():
    shape = SWEEP["split_keys_d8_r5"][:9] + (1,)
    d = dims_of(shape)
    _case(f"mlp_ring_bwd {d}")
    inp = inputs_for(shape, 0.02, 101)
    gpu, ref, _ = _run(d, inp, "bf16")
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        _check(k, gpu[k], ref[k])


# The MLP of the Llama-7B-like 8K layer at full size (1024 rows, hidden 4096,
# 8 shards of 1376): every element of dx and of the three weight gradients.
def test_mlp_ring_bwd_full_size_llama7b():
    wl = synth.WORKLOADS["llama7b_s8k_d8"]
    d = wl.dims
    _case("mlp_ring_bwd llama7b_s8k_d8 full size (all 1024 rows, all weight gradients)")
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    gpu, ref, _ = _run(d, inp, "bf16")
    for k in ("dx", "dw_g", "dw_u", "dw_d"):
        _check(k, gpu[k], ref[k])


def _keep_vs_recompute(d, inp, xdt, sample_rows=None):
    """tsp_mlp_ring_fwd_keep then tsp_mlp_ring_bwd_kept on rank d.rank's rows,
    beside tsp_mlp_ring_fwd then tsp_mlp_ring_bwd on the same inputs: y and
    every backward output must agree bit for bit; the kept g and u are held
    to the oracle's (all rows, or sample_rows of them)."""
    gpu, _, (xt, dyt, w, _, kw, _, _, _, _) = _run(d, inp, xdt)
    T, F, h = d.seq // d.degree, d.ffn, d.hidden
    M = d.batch * T
    f32 = dict(dtype=torch.float32, device="cuda")
    resid = torch.from_numpy(synth.make_grad(d, 3)[:, :T].copy()).cuda()
    y_ref, y = torch.empty_like(resid), torch.empty_like(resid)
    ws = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_MLP), dtype=torch.uint8, device="cuda")
    B.tsp_mlp_ring_fwd(d, xt, w["w_gate"], w["w_up"], w["w_down"], y_ref, ws, residual=resid, **kw)
    gu = torch.full((B.tsp_workspace_bytes(d, B.TSP_FN_GU) // 4,), float("nan"), **f32)
    B.tsp_mlp_ring_fwd_keep(d, xt, w["w_gate"], w["w_up"], w["w_down"], y, gu, ws, residual=resid, **kw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    dx = torch.empty_like(dyt)
    dwg, dwu = torch.empty((F, h), **f32), torch.empty((F, h), **f32)
    dwd = torch.empty((d.degree, h, F // d.degree), **f32)
    wsk = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_MLP_BWD_KEPT), dtype=torch.uint8, device="cuda")
    B.tsp_mlp_ring_bwd_kept(d, xt, dyt, w["w_gate"], w["w_up"], w["w_down"], gu, dx, dwg, dwu, dwd, wsk,
                            dx_residual=dyt, **kw)
    torch.cuda.synchronize()
    for k, v in (("dx", dx), ("dw_g", dwg), ("dw_u", dwu), ("dw_d", dwd)):
        assert np.array_equal(v.cpu().numpy(), gpu[k]), k
    # the kept g = x Wg^T and u = x Wu^T against the oracle's, from x as the
    # matrix cores saw it (f32 input: rounded to f16)
    x64 = xt.view(torch.bfloat16).double().cpu().numpy() if xdt == "bf16" else \
        xt.to(torch.float16).double().cpu().numpy()
    x64 = x64.reshape(M, h)
    rows = np.arange(M) if sample_rows is None else \
        np.sort(np.random.default_rng(5).choice(M, sample_rows, replace=False))
    wts = {n: orc.bf16_bits_to_f64(inp[n]) for n in ("w_g", "w_u", "w_d")}
    ref = bwd.mlp_backward(x64[rows], wts["w_g"], wts["w_u"], wts["w_d"], np.zeros((len(rows), h)))
    g_u = gu.view(2, M, F).cpu().numpy()
    _check("g", g_u[0][rows], ref["g"])
    _check("u", g_u[1][rows], ref["u"])


# tsp_mlp_ring_fwd_keep + tsp_mlp_ring_bwd_kept (g and u kept instead of
# recomputed): the forward's gate/up product and the backward's
# recomputation run the same kernel, and the kept epilogue of dA = dy W_down
# applies the recomputing epilogue's arithmetic to the same values, so y and
# every gradient agree bit for bit with tsp_mlp_ring_fwd + tsp_mlp_ring_bwd
# (held to the oracle above).  Shapes: the tiny layer, shards of 176 columns
# (ragged K segments), B = 2 with 96-position chunks, D = 1, a wider hidden
# size; every input type.
@pytest.mark.parametrize("name", ["tiny_d2", "ffn_tail_d4_r3", "gqa8_b2_c96", "d1", "wide_tiles_dh128"])
@pytest.mark.parametrize("xdt", ["bf16", "f16", "f32"])
def test_mlp_kept_equals_recompute(name, xdt):
    d, sigma, seed = _shape(name)
    _case(f"mlp kept vs recompute {name} x={xdt}")
    _keep_vs_recompute(d, inputs_for(d.astuple(), sigma, seed), xdt)


# The same with the transposed copy of W_down (TSP_TUNE_BWD_WEIGHTS = 1):
# the kept epilogue on the other dA kernel.
@pytest.mark.parametrize("name", ["tiny_d2", "ffn_tail_d4_r3"])
def test_mlp_kept_equals_recompute_weight_copies(name):
    d, sigma, seed = _shape(name)
    _case(f"mlp kept vs recompute {name} transposed weight copies")
    with tuning(bwd_weights=1):
        _keep_vs_recompute(d, inputs_for(d.astuple(), sigma, seed), "f32")


# The 8K layer's MLP at full size (1024 rows, 8 shards of 1376): bit equality
# of every output; g and u on 64 sampled rows against the oracle.
def test_mlp_kept_equals_recompute_full_size_llama7b():
    wl = synth.WORKLOADS["llama7b_s8k_d8"]
    _case("mlp kept vs recompute llama7b_s8k_d8 full size")
    _keep_vs_recompute(wl.dims, synth.make_inputs(wl.dims, wl.sigma, wl.seed), "f16", sample_rows=64)
