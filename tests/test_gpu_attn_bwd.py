"""GPU parity of the attention backward (tsp_attn_bwd and tsp_attn_bwd_proj,
through the C ABI) against the float64 backward oracle.

Every rank's tsp_attn_bwd runs on the one GPU; their K/V-gradient send
buffers are then summed for the checked rank (the reduce-scatter, simulated
here as the all-gather is simulated by tsp_qkv_proj for the other ranks) and
fed to tsp_attn_bwd_proj.  References: the oracle's rank_attention_backward
(every rank's queries' share, the reduce-scatter sum, the projection share).
Bars, relative to each output: max-abs over the largest reference element <=
2e-2 and relative Frobenius <= 5e-3, as for the MLP backward.
"""
import dataclasses

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


def _check(name, got, ref):
    ma, rf = errors(got, ref)
    ma_rel = ma / max(float(np.abs(ref).max()), 1e-30)
    print(f"  {name}: max_abs/max={ma_rel:.3e} rel_frob={rf:.3e}", flush=True)
    assert np.all(np.isfinite(got)), name
    assert ma_rel <= MAX_ABS and rf <= REL_FROB, (name, ma_rel, rf)


class _Ranks:
    """Device weights, every rank's bf16 rows and the filled all-gathered K/V."""

    def __init__(self, d, inp):
        self.d = d
        self.w = {k: v.cuda() for k, v in pack_weights(inp, d).items()}
        self.l2g = [orc.local_to_global(d.seq, d.degree, r, d.partition) for r in range(d.degree)]
        self.x_loc = [torch.from_numpy(np.ascontiguousarray(inp["x"][:, self.l2g[r]]).view(np.int16)).cuda()
                      for r in range(d.degree)]
        nkv = B.tsp_workspace_bytes(d, B.TSP_FN_KV_GATHERED) // 2
        self.kv = torch.zeros(nkv, dtype=torch.int16, device="cuda")
        for r in range(d.degree):
            B.tsp_qkv_proj(self.rank(r), r, self.x_loc[r], self.w["w_qkv"], None, self.kv)
        # the attention's work plan (and so its scratch) depends on the rank
        n1 = max(B.tsp_workspace_bytes(self.rank(r), B.TSP_FN_ATTN_BWD) for r in range(d.degree))
        self.ws1 = torch.empty(n1, dtype=torch.uint8, device="cuda")
        self.ws2 = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_ATTN_BWD_PROJ), dtype=torch.uint8,
                               device="cuda")

    def rank(self, r):
        return dataclasses.replace(self.d, rank=r)

    def bwd(self, r, dh_rows):
        """tsp_attn_bwd on rank r: (dq, dkv_send, dw_o) device tensors."""
        d = self.rank(r)
        T = d.seq // d.degree
        dq = torch.empty((d.batch, T, d.n_q_heads * d.head_dim), dtype=torch.float32, device="cuda")
        send = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_DKV) // 4, dtype=torch.float32, device="cuda")
        dwo = torch.empty((d.degree, d.hidden, d.n_q_heads // d.degree * d.head_dim), dtype=torch.float32,
                          device="cuda")
        B.tsp_attn_bwd(d, self.x_loc[r], self.w["w_qkv"], self.w["w_o"], self.kv, dh_rows, dq, send, dwo, self.ws1)
        return dq, send, dwo

    def proj(self, r, dq, own, dx_residual):
        d = self.rank(r)
        T = d.seq // d.degree
        dx = torch.empty((d.batch, T, d.hidden), dtype=torch.float32, device="cuda")
        nqkv = (d.n_q_heads + 2 * d.n_kv_heads) // d.degree * d.head_dim
        dwqkv = torch.empty((d.degree, nqkv, d.hidden), dtype=torch.float32, device="cuda")
        B.tsp_attn_bwd_proj(d, self.x_loc[r], self.w["w_qkv"], dq, own, dx, dwqkv, self.ws2,
                            dx_residual=dx_residual)
        return dx, dwqkv


def _send_ref(d, contrib, l2g):
    """The oracle's contribution [D j][2][B][S][kvd] laid out as the send
    buffer [D dst][D j][2][B][T][kvd]."""
    return np.stack([contrib[:, :, :, l2g[g]] for g in range(d.degree)])


def _dwo_ref(d, dw_o):
    qs = d.n_q_heads // d.degree * d.head_dim
    return np.stack([dw_o[:, j * qs:(j + 1) * qs] for j in range(d.degree)])


def _run_case(d, inp, seed=11):
    R = _Ranks(d, inp)
    D, T = d.degree, d.seq // d.degree
    dh_all = synth.make_grad(dataclasses.replace(d, rank=0), seed)     # [B][S][h] float32
    # per-rank phase 1
    outs = []
    for rq in range(D):
        dh_rows = torch.from_numpy(np.ascontiguousarray(dh_all[:, R.l2g[rq]])).cuda()
        outs.append(R.bwd(rq, dh_rows) + (dh_rows,))
    torch.cuda.synchronize()
    r = d.rank
    per = 2 * d.batch * T * (d.n_kv_heads // D) * d.head_dim * D     # floats per destination block
    own = sum(o[1][r * per:(r + 1) * per] for o in outs)              # the reduce-scatter (test plumbing)
    dq, send, dwo, dh_rows = outs[r]
    dx, dwqkv = R.proj(r, dq, own.contiguous(), dh_rows)
    torch.cuda.synchronize()
    ref = bwd.rank_attention_backward(inp, d, dh_all)
    kvd = d.n_kv_heads // D * d.head_dim
    _check("dq", dq.cpu().numpy(), ref["dq"])
    _check("dkv_send", send.cpu().numpy().reshape(D, D, 2, d.batch, T, kvd), _send_ref(d, ref["dkv_contrib"], R.l2g))
    _check("dw_o", dwo.cpu().numpy(), _dwo_ref(d, ref["dw_o"]))
    _check("dkv_own", own.cpu().numpy().reshape(D, 2, d.batch, T, kvd), ref["dkv_own"])
    _check("dx", dx.cpu().numpy(), ref["dx_attn"] + dh_all[:, R.l2g[r]])
    _check("dw_qkv", dwqkv.cpu().numpy(), ref["dw_qkv"])
    return R, outs


# Shapes: MHA and GQA 2/4/8, head_dim 64 and 128, B = 2, D = 1, one-row
# chunks (c = 1), chunks that are not multiples of 64 (c = 24, 80, 96), and
# row blocks long enough that dQ is cut into key pieces (split_keys_*).
SHAPES = ["mha_d2_r1", "gqa4_dh128_d4_r2", "gqa8_b2_c96", "d1", "c1_d8_r5", "c24_generic_reorder",
          "gqa2_b2_dh128_c80", "split_keys_dh128", "split_keys_gqa_b2", "split_keys_d8_r5"]


@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
@pytest.mark.parametrize("name", SHAPES)
def test_attn_bwd(name, partition):
    shape = SWEEP[name][:9] + (partition,)
    d = dims_of(shape)
    _case(f"attn_bwd {name} partition={partition} {d}")
    inp = inputs_for(shape, 0.02, 101)
    _run_case(d, inp)


def test_attn_bwd_tiny_layer_and_determinism():
    wl = synth.WORKLOADS["tiny_d2"]
    d = wl.dims
    _case(f"attn_bwd tiny_d2 twice {d}")
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    R, outs = _run_case(d, inp)
    # a second run on the same inputs repeats every output bit for bit
    dq, send, dwo, dh_rows = outs[d.rank]
    dq2, send2, dwo2 = R.bwd(d.rank, dh_rows)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(send, send2) and torch.equal(dwo, dwo2)


# dO = dh W_O and dx = G W_QKV read the weights as stored (K-major
# products); TSP_TUNE_BWD_WEIGHTS = 1 multiplies by transposed copies held in
# the workspaces.  Same K order, so the outputs agree bit for bit.
@pytest.mark.parametrize("name", ["gqa4_dh128_d4_r2", "c24_generic_reorder"])
def test_attn_bwd_weight_copies_match_kmajor(name):
    shape = SWEEP[name][:9] + (0,)
    d = dims_of(shape)
    _case(f"attn_bwd {name} weights as stored vs transposed copies {d}")
    inp = inputs_for(shape, 0.02, 101)
    R = _Ranks(d, inp)
    r = d.rank
    dh_rows = torch.from_numpy(np.ascontiguousarray(synth.make_grad(d, 13)[:, R.l2g[r]])).cuda()
    own = torch.randn(B.tsp_workspace_bytes(d, B.TSP_FN_DKV) // 4 // d.degree, device="cuda") * 0.05
    outs = []
    for knob in (None, 1):
        with tuning(bwd_weights=knob):
            n1 = B.tsp_workspace_bytes(d, B.TSP_FN_ATTN_BWD)
            n2 = B.tsp_workspace_bytes(d, B.TSP_FN_ATTN_BWD_PROJ)
            R.ws1 = torch.empty(n1, dtype=torch.uint8, device="cuda")
            R.ws2 = torch.empty(n2, dtype=torch.uint8, device="cuda")
            dq, send, dwo = R.bwd(r, dh_rows)
            dx, dwqkv = R.proj(r, dq, own, dh_rows)
            torch.cuda.synchronize()
            outs.append((n1, n2, dq, send, dwo, dx, dwqkv))
    (a1, a2, *a), (b1, b2, *b) = outs
    assert b1 > a1 and b2 > a2  # the copies live in the workspaces
    for name_, x, y in zip(("dq", "dkv_send", "dw_o", "dx", "dw_qkv"), a, b):
        assert torch.equal(x, y), name_


@pytest.mark.parametrize("name", ["gqa4_dh128_d4_r2", "mha_d2_r1"])
def test_attn_bwd_sharp_softmax(name):
    # weights drawn with sigma 0.25 (as the forward's sharp-softmax test):
    # scores spread over tens of units, so softmax rows are nearly one-hot
    # and dS is large on a few keys
    shape = SWEEP[name][:9] + (0,)
    d = dims_of(shape)
    _case(f"attn_bwd {name} sharp softmax {d}")
    _run_case(d, inputs_for(shape, 0.25, 103))


# Full size, the Llama-7B-like 8K layer on rank 0 of 8: tsp_attn_bwd against the
# oracle's share of rank 0's queries (every element of dq, dw_o and the whole
# send buffer), and tsp_attn_bwd_proj on seeded synthetic dq and dkv_own (so
# that its check needs no other rank's share) against the oracle's projection.
def test_attn_bwd_full_size_llama7b():
    wl = synth.WORKLOADS["llama7b_s8k_d8"]
    d = wl.dims
    _case("attn_bwd llama7b_s8k_d8 full size, rank 0")
    inp = synth.make_inputs(d, wl.sigma, wl.seed)
    R = _Ranks(d, inp)
    D, T = d.degree, d.seq // d.degree
    dh_rows = synth.make_grad(d, 11)[:, R.l2g[d.rank]]
    dh_t = torch.from_numpy(np.ascontiguousarray(dh_rows)).cuda()
    dq, send, dwo = R.bwd(d.rank, dh_t)
    torch.cuda.synchronize()
    ref = bwd.rank_attention_bwd_queries(inp, d, dh_rows)
    kvd = d.n_kv_heads // D * d.head_dim
    _check("dq", dq.cpu().numpy(), ref["dq"])
    _check("dkv_send", send.cpu().numpy().reshape(D, D, 2, d.batch, T, kvd), _send_ref(d, ref["dkv_contrib"], R.l2g))
    _check("dw_o", dwo.cpu().numpy(), _dwo_ref(d, ref["dw_o"]))
    rng = np.random.default_rng(17)
    dq_in = rng.standard_normal(dq.shape).astype(np.float32) * 0.05
    own_in = rng.standard_normal((D, 2, d.batch, T, kvd)).astype(np.float32) * 0.05
    dx, dwqkv = R.proj(d.rank, torch.from_numpy(dq_in).cuda(), torch.from_numpy(own_in).cuda(), dh_t)
    torch.cuda.synchronize()
    pref = bwd.rank_attention_bwd_proj(inp, d, dq_in, own_in)
    _check("dx", dx.cpu().numpy(), pref["dx_attn"] + dh_rows)
    _check("dw_qkv", dwqkv.cpu().numpy(), pref["dw_qkv"])


# tsp_attn_fwd_keep + tsp_attn_bwd_kept (the forward's Q, O and row
# normalisers kept instead of recomputed) against tsp_attn_fwd +
# tsp_attn_bwd: the same kernels produce the kept tensors, so the layer
# output and every backward output agree bit for bit.  Shapes: GQA 4 with
# head_dim 128 under both partitions, blocks cut into key pieces (the merge
# writes those rows' normalisers), chunks of 24 positions, the 8K layer.
@pytest.mark.parametrize("name,partition", [("gqa4_dh128_d4_r2", 0), ("gqa4_dh128_d4_r2", 1),
                                            ("split_keys_dh128", 0), ("c24_generic_reorder", 1),
                                            ("llama7b_s8k_d8", 0)])
def test_attn_bwd_kept_equals_recompute(name, partition):
    if name in synth.WORKLOADS:
        wl = synth.WORKLOADS[name]
        d = dataclasses.replace(wl.dims, partition=partition)
        inp = synth.make_inputs(d, wl.sigma, wl.seed)
    else:
        shape = SWEEP[name][:9] + (partition,)
        d = dims_of(shape)
        inp = inputs_for(shape, 0.02, 101)
    _case(f"attn_bwd_kept {name} partition={partition} {d}")
    R = _Ranks(d, inp)
    r = d.rank
    T = d.seq // d.degree
    f32 = dict(dtype=torch.float32, device="cuda")
    x32 = R.x_loc[r].view(torch.bfloat16).float()
    out_ref = torch.empty((d.batch, T, d.hidden), **f32)
    wsa = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_ATTN), dtype=torch.uint8, device="cuda")
    B.tsp_attn_fwd(d, R.x_loc[r], R.w["w_qkv"], R.w["w_o"], R.kv, out_ref, wsa, residual=x32)
    qd = d.n_q_heads * d.head_dim
    out = torch.empty_like(out_ref)
    q_keep = torch.empty(d.batch * T * qd, dtype=torch.int16, device="cuda")
    o_keep = torch.empty_like(q_keep)
    lse = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_LSE) // 4, **f32)
    wsk = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_ATTN_KEEP), dtype=torch.uint8, device="cuda")
    B.tsp_attn_fwd_keep(d, R.x_loc[r], R.w["w_qkv"], R.w["w_o"], R.kv, out, q_keep, o_keep, lse, wsk, residual=x32)
    torch.cuda.synchronize()
    assert torch.equal(out, out_ref)
    dh_rows = torch.from_numpy(np.ascontiguousarray(synth.make_grad(d, 29)[:, R.l2g[r]])).cuda()
    dq, send, dwo = R.bwd(r, dh_rows)
    dq2, send2, dwo2 = torch.empty_like(dq), torch.empty_like(send), torch.empty_like(dwo)
    wsb = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_ATTN_BWD_KEPT), dtype=torch.uint8, device="cuda")
    B.tsp_attn_bwd_kept(d, R.w["w_o"], R.kv, q_keep, o_keep, lse, dh_rows, dq2, send2, dwo2, wsb)
    torch.cuda.synchronize()
    for nm, x, y in (("dq", dq, dq2), ("dkv_send", send, send2), ("dw_o", dwo, dwo2)):
        assert torch.equal(x, y), nm
