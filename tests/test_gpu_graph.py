"""GPU: the layer forward and the backward calls captured into HIP graphs
(torch.cuda.CUDAGraph on the calls' stream) and replayed.

The library enqueues kernels only (no allocation, memset, copy or
synchronisation inside a call), so a caller can capture a whole layer step and
replay it without per-call launch work.  Every replay is checked against the
eager call bit for bit, with eager work and synchronisations between the
replays, and a replay after the inputs changed in place must give the eager
result for the new inputs (the graph reads its inputs at replay time).
"""
import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_amd import binding as B
from folded_tensor_sequence_amd.harness import RankProblem

from gpu_util import SWEEP, dims_of, inputs_for

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _capture(fn):
    """Warm-up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _problem(name):
    if name in synth.WORKLOADS:
        wl = synth.WORKLOADS[name]
        return wl.dims, synth.make_inputs(wl.dims, wl.sigma, wl.seed)
    shape = SWEEP[name]
    return dims_of(shape), inputs_for(shape, 0.02, 101)


# The layer forward: small layers with split key pieces and ragged tiles, and
# the 8K layer the benchmark times.
@pytest.mark.parametrize("name", ["mha_d2_r1", "split_keys_d8_r5", "ffn_tail_d4_r3", "llama7b_s8k_d8"])
def test_layer_fwd_graph_replay(name):
    d, inp = _problem(name)
    print(f"[case] layer_fwd graph replay {name} {d}", flush=True)
    prob = RankProblem.build(d, inp)
    y_ref = prob.layer().clone()
    # the eager result for other inputs: x_local with its rows reversed
    x_ref = prob.x_local.clone()
    prob.x_local.copy_(torch.flip(x_ref, dims=[1]))
    y_flip = prob.layer().clone()
    prob.x_local.copy_(x_ref)
    torch.cuda.synchronize()
    g = _capture(prob.layer)
    other = torch.randn(1 << 20, device="cuda")
    for i in range(3):
        prob.y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(prob.y, y_ref), f"replay {i}"
        # eager work between replays (library and torch kernels)
        prob.layer()
        other.mul_(1.0001).sum().item()
        assert torch.equal(prob.y, y_ref)
    prob.x_local.copy_(torch.flip(x_ref, dims=[1]))
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(prob.y, y_flip)
    prob.x_local.copy_(x_ref)
    if name == "llama7b_s8k_d8":
        # eager calls against replays (informational: the difference is a few
        # microseconds and varies with the conditions)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        for _ in range(5):
            prob.layer()
            g.replay()
        ev[0].record()
        for _ in range(20):
            prob.layer()
        ev[1].record()
        for _ in range(20):
            g.replay()
        ev[2].record()
        torch.cuda.synchronize()
        print(f"  eager {ev[0].elapsed_time(ev[1]) / 20 * 1e3:.1f} us per layer, "
              f"graph replay {ev[1].elapsed_time(ev[2]) / 20 * 1e3:.1f} us", flush=True)


# The backward calls of one rank in one graph: the MLP ring's backward, part 1
# of the attention backward (and its kept-activation form), part 2.
@pytest.mark.parametrize("name", ["gqa4_dh128_d4_r2", "split_keys_d8_r5"])
def test_backward_graph_replay(name):
    d, inp = _problem(name)
    print(f"[case] backward graph replay {name} {d}", flush=True)
    prob = RankProblem.build(d, inp)
    B.tsp_qkv_proj(d, d.rank, prob.x_local, prob.w["w_qkv"], None, prob.kv_gathered)
    w = prob.w
    D, T, h, F = d.degree, d.seq // d.degree, d.hidden, d.ffn
    qd = d.n_q_heads * d.head_dim
    nqkv = (d.n_q_heads + 2 * d.n_kv_heads) // D * d.head_dim
    f32 = dict(dtype=torch.float32, device="cuda")
    l2g = prob.l2g[d.rank].cpu().numpy()
    dy = torch.from_numpy(np.ascontiguousarray(synth.make_grad(d, 11)[:, l2g])).cuda()
    outs = {
        "dxm": torch.empty_like(dy), "dwg": torch.empty((F, h), **f32), "dwu": torch.empty((F, h), **f32),
        "dwd": torch.empty((D, h, F // D), **f32), "dq": torch.empty((d.batch, T, qd), **f32),
        "send": torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_DKV) // 4, **f32),
        "dwo": torch.empty((D, h, qd // D), **f32), "dx": torch.empty_like(dy),
        "dwqkv": torch.empty((D, nqkv, h), **f32), "dq_k": torch.empty((d.batch, T, qd), **f32),
        "send_k": torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_DKV) // 4, **f32),
        "dwo_k": torch.empty((D, h, qd // D), **f32),
    }
    per = outs["send"].numel() // D
    own = outs["send"][d.rank * per:(d.rank + 1) * per]
    ws = {fn: torch.empty(B.tsp_workspace_bytes(d, fn), dtype=torch.uint8, device="cuda")
          for fn in (B.TSP_FN_MLP_BWD, B.TSP_FN_ATTN_BWD, B.TSP_FN_ATTN_BWD_PROJ, B.TSP_FN_ATTN_KEEP,
                     B.TSP_FN_ATTN_BWD_KEPT)}
    q_keep = torch.empty(d.batch * T * qd, dtype=torch.int16, device="cuda")
    o_keep = torch.empty_like(q_keep)
    lse = torch.empty(B.tsp_workspace_bytes(d, B.TSP_FN_LSE) // 4, **f32)
    hout = torch.empty_like(dy)
    B.tsp_attn_fwd_keep(d, prob.x_local, w["w_qkv"], w["w_o"], prob.kv_gathered, hout, q_keep, o_keep, lse,
                        ws[B.TSP_FN_ATTN_KEEP])
    o = outs

    def step():
        B.tsp_mlp_ring_bwd(d, prob.x_local, dy, w["w_gate"], w["w_up"], w["w_down"], o["dxm"], o["dwg"], o["dwu"],
                           o["dwd"], ws[B.TSP_FN_MLP_BWD], dx_residual=dy, x_dtype=B.TSP_BF16)
        B.tsp_attn_bwd(d, prob.x_local, w["w_qkv"], w["w_o"], prob.kv_gathered, dy, o["dq"], o["send"], o["dwo"],
                       ws[B.TSP_FN_ATTN_BWD])
        B.tsp_attn_bwd_kept(d, w["w_o"], prob.kv_gathered, q_keep, o_keep, lse, dy, o["dq_k"], o["send_k"],
                            o["dwo_k"], ws[B.TSP_FN_ATTN_BWD_KEPT])
        B.tsp_attn_bwd_proj(d, prob.x_local, w["w_qkv"], o["dq"], own, o["dx"], o["dwqkv"],
                            ws[B.TSP_FN_ATTN_BWD_PROJ], dx_residual=dy)

    step()
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    for k in ("dq", "send", "dwo"):
        assert torch.equal(ref[k], ref[k + "_k"]), k
    g = _capture(step)
    for i in range(3):
        for v in outs.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(v, ref[k]), (i, k)
        step()
        torch.cuda.synchronize()
