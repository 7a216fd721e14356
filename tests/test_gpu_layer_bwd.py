"""GPU: the whole TSP layer backward, composed from the C ABI's pieces on
every rank of small layers, against the unsharded layer's gradients.

For each rank r: the attention forward (h = x + Attn(x), the MLP's input),
tsp_mlp_ring_bwd (dh = dy + the MLP branch's input gradient, the rank's
weight-gradient contributions), tsp_attn_bwd (dQ, the K/V-gradient send
buffer, dW_O share); then the reduce-scatter (test plumbing: the blocks for
rank r summed over ranks) and tsp_attn_bwd_proj (dx = dh + the attention
branch's input gradient, dW_QKV share).  With kept activations the forward
calls also hand over what the backward would recompute (tsp_attn_fwd_keep:
Q, O, the row normalisers; tsp_mlp_ring_fwd_keep: g and u) and the backward
calls take them (tsp_attn_bwd_kept, tsp_mlp_ring_bwd_kept).  Reference: the oracle's
layer_backward (float64 autograd-free gradients of the unsharded layer over
whole sequences, pinned on the CPU against torch autograd and finite
differences): every rank's dh and dx rows, and the weight gradients summed
over ranks, in the ABI layouts.  Bars as for the other backward tests,
relative to each gradient: max-abs over its largest element <= 2e-2,
relative Frobenius <= 5e-3.
"""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_amd import binding as B
from folded_tensor_sequence_amd.harness import RankProblem
from oracle import tsp_backward as bwd

from gpu_util import MAX_ABS, REL_FROB, SWEEP, dims_of, errors, inputs_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _check(name, got, ref):
    ma, rf = errors(got, ref)
    ma_rel = ma / max(float(np.abs(ref).max()), 1e-30)
    print(f"  {name}: max_abs/max={ma_rel:.3e} rel_frob={rf:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert ma_rel <= MAX_ABS and rf <= REL_FROB, (name, ma_rel, rf)


def _layer_backward_on_gpu(d, inp, dy, kept=False):
    """Every rank's pieces; returns per-rank dh, dx rows and the summed weight
    gradients (ABI layouts), as numpy.  kept: the forward's activations kept
    instead of recomputed."""
    prob = RankProblem.build(d, inp)
    w = prob.w
    D, T, h = d.degree, d.seq // d.degree, d.hidden
    F, qd = d.ffn, d.n_q_heads * d.head_dim
    qs, nqkv = qd // D, (d.n_q_heads + 2 * d.n_kv_heads) // D * d.head_dim
    ranks = [dataclasses.replace(d, rank=r) for r in range(D)]
    xloc = [prob.x_full.index_select(1, prob.l2g[r].long()).contiguous() for r in range(D)]
    f32 = dict(dtype=torch.float32, device="cuda")
    dwg, dwu = torch.zeros((F, h), **f32), torch.zeros((F, h), **f32)
    dwd, dwo = torch.zeros((D, h, F // D), **f32), torch.zeros((D, h, qs), **f32)
    dwqkv = torch.zeros((D, nqkv, h), **f32)
    # every rank's K/V slot of the all-gather (the build skipped dims.rank's:
    # the layer call writes it), so that each rank's attention sees all keys
    B.tsp_qkv_proj(d, d.rank, xloc[d.rank], w["w_qkv"], None, prob.kv_gathered)
    dhs, dqs, sends, keeps = [], [], [], []
    for r, dr in enumerate(ranks):
        # forward to the MLP input h
        x32 = xloc[r].view(torch.bfloat16).float()
        hr = torch.empty((d.batch, T, h), **f32)
        if kept:
            q_keep = torch.empty(d.batch * T * qd, dtype=torch.int16, device="cuda")
            o_keep = torch.empty_like(q_keep)
            lse = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_LSE) // 4, **f32)
            wsa = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_ATTN_KEEP), dtype=torch.uint8, device="cuda")
            B.tsp_attn_fwd_keep(dr, xloc[r], w["w_qkv"], w["w_o"], prob.kv_gathered, hr, q_keep, o_keep, lse, wsa,
                                residual=x32)
            keeps.append((q_keep, o_keep, lse))
        else:
            wsa = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_ATTN), dtype=torch.uint8, device="cuda")
            B.tsp_attn_fwd(dr, xloc[r], w["w_qkv"], w["w_o"], prob.kv_gathered, hr, wsa, residual=x32)
        l2g = prob.l2g[r].cpu().numpy()
        dyr = torch.from_numpy(np.ascontiguousarray(dy[:, l2g])).cuda()
        dhr = torch.empty_like(dyr)
        g, u, dd = torch.empty_like(dwg), torch.empty_like(dwu), torch.empty_like(dwd)
        if kept:
            # the MLP forward (its output is not needed here) keeps g and u
            gu = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_GU) // 4, **f32)
            wsf = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_MLP), dtype=torch.uint8, device="cuda")
            B.tsp_mlp_ring_fwd_keep(dr, hr, w["w_gate"], w["w_up"], w["w_down"], torch.empty_like(hr), gu, wsf,
                                    x_dtype=B.TSP_F32)
            wsm = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_MLP_BWD_KEPT), dtype=torch.uint8, device="cuda")
            B.tsp_mlp_ring_bwd_kept(dr, hr, dyr, w["w_gate"], w["w_up"], w["w_down"], gu, dhr, g, u, dd, wsm,
                                    dx_residual=dyr, x_dtype=B.TSP_F32)
        else:
            wsm = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_MLP_BWD), dtype=torch.uint8, device="cuda")
            B.tsp_mlp_ring_bwd(dr, hr, dyr, w["w_gate"], w["w_up"], w["w_down"], dhr, g, u, dd, wsm,
                               dx_residual=dyr, x_dtype=B.TSP_F32)
        dwg += g
        dwu += u
        dwd += dd
        dhs.append(dhr)
    torch.cuda.synchronize()
    for r, dr in enumerate(ranks):
        dq = torch.empty((d.batch, T, qd), **f32)
        send = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_DKV) // 4, **f32)
        o = torch.empty((D, h, qs), **f32)
        if kept:
            ws1 = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_ATTN_BWD_KEPT), dtype=torch.uint8, device="cuda")
            B.tsp_attn_bwd_kept(dr, w["w_o"], prob.kv_gathered, *keeps[r], dhs[r], dq, send, o, ws1)
        else:
            ws1 = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_ATTN_BWD), dtype=torch.uint8, device="cuda")
            B.tsp_attn_bwd(dr, xloc[r], w["w_qkv"], w["w_o"], prob.kv_gathered, dhs[r], dq, send, o, ws1)
        dwo += o
        dqs.append(dq)
        sends.append(send)
    torch.cuda.synchronize()
    per = sends[0].numel() // D
    dxs = []
    for r, dr in enumerate(ranks):
        own = sum(sd[r * per:(r + 1) * per] for sd in sends).contiguous()  # the reduce-scatter
        dx = torch.empty((d.batch, T, h), **f32)
        q = torch.empty((D, nqkv, h), **f32)
        ws2 = torch.empty(B.tsp_workspace_bytes(dr, B.TSP_FN_ATTN_BWD_PROJ), dtype=torch.uint8, device="cuda")
        B.tsp_attn_bwd_proj(dr, xloc[r], w["w_qkv"], dqs[r], own, dx, q, ws2, dx_residual=dhs[r])
        dwqkv += q
        dxs.append(dx)
    torch.cuda.synchronize()
    l2gs = [prob.l2g[r].cpu().numpy() for r in range(D)]
    out = {"dh": [t.cpu().numpy() for t in dhs], "dx": [t.cpu().numpy() for t in dxs], "l2g": l2gs}
    out.update({k: v.cpu().numpy() for k, v in
                (("dw_g", dwg), ("dw_u", dwu), ("dw_d", dwd), ("dw_o", dwo), ("dw_qkv", dwqkv))})
    return out


# The tiny layer (D = 2); GQA 4 with head_dim 128 at D = 4; chunks of 24
# positions (not multiples of 64) at D = 2; MHA at D = 2 with a 768-wide FFN.
CASES = [("tiny_d2", 0), ("gqa4_dh128_d4_r2", 0), ("gqa4_dh128_d4_r2", 1), ("c24_generic_reorder", 1),
         ("mha_d2_r1", 0)]


def _case(name, partition):
    if name in synth.WORKLOADS:
        wl = synth.WORKLOADS[name]
        d = dataclasses.replace(wl.dims, partition=partition)
        inp = synth.make_inputs(d, wl.sigma, wl.seed)
    else:
        shape = SWEEP[name][:9] + (partition,)
        d = dims_of(shape)
        inp = inputs_for(shape, 0.02, 101)
    return d, inp


@pytest.mark.parametrize("name,partition", CASES)
def test_layer_backward_composed_equals_unsharded(name, partition):
    d, inp = _case(name, partition)
    print(f"[case] composed layer backward {name} partition={partition} {d}", flush=True)
    dy = synth.make_grad(d, 23)
    _check_against_oracle(d, inp, dy, _layer_backward_on_gpu(d, inp, dy))


# The same composition with the forward's activations kept (attention: Q, O,
# row normalisers; MLP: g and u): the oracle's bars, and every output equal
# bit for bit to the recomputing composition's.
@pytest.mark.parametrize("name,partition", [("tiny_d2", 0), ("gqa4_dh128_d4_r2", 1), ("c24_generic_reorder", 1)])
def test_layer_backward_composed_kept(name, partition):
    d, inp = _case(name, partition)
    print(f"[case] composed layer backward, kept activations, {name} partition={partition} {d}", flush=True)
    dy = synth.make_grad(d, 23)
    got = _layer_backward_on_gpu(d, inp, dy, kept=True)
    _check_against_oracle(d, inp, dy, got)
    rec = _layer_backward_on_gpu(d, inp, dy)
    for k in ("dh", "dx"):
        for r in range(d.degree):
            assert np.array_equal(got[k][r], rec[k][r]), (k, r)
    for k in ("dw_g", "dw_u", "dw_d", "dw_o", "dw_qkv"):
        assert np.array_equal(got[k], rec[k]), k


def _check_against_oracle(d, inp, dy, got):
    ref = bwd.layer_backward(inp, d, dy)
    D = d.degree
    qs = d.n_q_heads // D * d.head_dim
    hq, hkv, dh = d.n_q_heads // D, d.n_kv_heads // D, d.head_dim
    fs = d.ffn // D
    _check("dh", np.concatenate(got["dh"], axis=1),
           np.concatenate([ref["dh"][:, l] for l in got["l2g"]], axis=1))
    _check("dx", np.concatenate(got["dx"], axis=1),
           np.concatenate([ref["dx"][:, l] for l in got["l2g"]], axis=1))
    _check("dw_gate", got["dw_g"], ref["dw_g"])
    _check("dw_up", got["dw_u"], ref["dw_u"])
    _check("dw_down", got["dw_d"], np.stack([ref["dw_d"][:, j * fs:(j + 1) * fs] for j in range(D)]))
    _check("dw_o", got["dw_o"], np.stack([ref["dw_o"][:, j * qs:(j + 1) * qs] for j in range(D)]))
    packed = np.stack([np.concatenate([ref["dw_q"][j * hq * dh:(j + 1) * hq * dh],
                                       ref["dw_k"][j * hkv * dh:(j + 1) * hkv * dh],
                                       ref["dw_v"][j * hkv * dh:(j + 1) * hkv * dh]]) for j in range(D)])
    _check("dw_qkv", got["dw_qkv"], packed)
