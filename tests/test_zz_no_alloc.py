"""tsp_layer_fwd_noalloc, the layer entry point that allocates nothing (its
workspace is the library's fixed scratch array), against tsp_layer_fwd on the
same inputs: two calls in a row on one GPU, the second with a smaller layer,
each bit-identical to tsp_layer_fwd (same kernels, same order) and, on the
tiny layer, within the parity bar of the float64 oracle on every row."""
import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_amd import binding as B
from folded_tensor_sequence_amd.harness import RankProblem
from oracle import tsp_oracle as orc

from gpu_util import assert_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()


def _noalloc(prob):
    w = prob.w
    y = torch.full_like(prob.y, float("nan"))
    B.tsp_layer_fwd_noalloc(prob.dims, prob.x_local, w["w_qkv"], w["w_o"], w["w_gate"], w["w_up"], w["w_down"],
                            prob.kv_gathered, y)
    torch.cuda.synchronize()
    return y


def test_noalloc_matches_layer_fwd_on_two_calls():
    for name in ("llama7b_s8k_d8", "tiny_d2"):          # the second call is the smaller one
        wl = synth.WORKLOADS[name]
        d = wl.dims
        print(f"[case] layer_fwd_noalloc {name}", flush=True)
        assert B.tsp_workspace_bytes(d, B.TSP_FN_LAYER) <= B.TSP_SCRATCH_BYTES
        inp = synth.make_inputs(d, wl.sigma, wl.seed)
        prob = RankProblem.build(d, inp)
        y_ref = prob.layer().clone()
        torch.cuda.synchronize()
        y = _noalloc(prob)
        assert torch.equal(y, y_ref), f"{name}: noalloc output differs from tsp_layer_fwd"
        if name == "tiny_d2":
            assert_close(y.cpu().numpy(), orc.layer_rank_rows(inp, d)["y"], what="noalloc y (tiny, every row)")
        del prob
        torch.cuda.empty_cache()


def test_noalloc_rejects_a_layer_beyond_the_scratch_array():
    wl = synth.WORKLOADS["llama3_8b_gqa_s16k_d8"]
    d = wl.dims
    need = B.tsp_workspace_bytes(d, B.TSP_FN_LAYER)
    assert need > B.TSP_SCRATCH_BYTES
    T = d.seq // d.degree
    # correctly sized (uninitialised) tensors: the size check fails before any launch
    z = B._Sizes(d)
    e16 = lambda n: torch.empty(n // 2, dtype=torch.int16, device="cuda")
    with pytest.raises(B.TspError) as ei:
        B.tsp_layer_fwd_noalloc(d, e16(z.x16), e16(z.w_qkv), e16(z.w_o), e16(z.w_ffn), e16(z.w_ffn), e16(z.w_ffn),
                                e16(B.tsp_workspace_bytes(d, B.TSP_FN_KV_GATHERED)),
                                torch.empty((d.batch, T, d.hidden), dtype=torch.float32, device="cuda"))
    assert ei.value.code == B.TSP_ERR_SCRATCH
