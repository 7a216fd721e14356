"""GPU: the C ABI driven from plain C++ (tests/abi_c_caller.cpp, built by
build() into tests/libtsp_c_caller.so): the caller includes only
include/tsp.h, allocates device memory with hipMalloc, fills the other
ranks' K/V slots with tsp_qkv_proj and runs tsp_layer_fwd.  Its output must
equal the Python binding's run of the same layer bit for bit (both call the
same library; the binding's run is held to the oracle by
tests/test_gpu_parity.py)."""
import ctypes
import dataclasses
import os

import numpy as np
import pytest
import torch

import synth
from folded_tensor_sequence_amd import binding as B
from folded_tensor_sequence_amd.harness import RankProblem, pack_weights

from gpu_util import SWEEP, dims_of, inputs_for

pytestmark = pytest.mark.gpu

CALLER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsp_c_caller.so")


@pytest.fixture(scope="module")
def caller():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load()
    assert os.path.exists(CALLER), "build() makes tests/libtsp_c_caller.so"
    lib = ctypes.CDLL(CALLER)
    lib.tsp_c_caller_run.argtypes = [ctypes.c_char_p]
    lib.tsp_c_caller_run.restype = ctypes.c_int
    return lib


def _problem(name, partition):
    if name in synth.WORKLOADS:
        wl = synth.WORKLOADS[name]
        d = dataclasses.replace(wl.dims, partition=partition)
        return d, synth.make_inputs(d, wl.sigma, wl.seed)
    shape = SWEEP[name][:9] + (partition,)
    return dims_of(shape), inputs_for(shape, 0.02, 101)


# The tiny layer; GQA 4 with head_dim 128 under the striped partition; rank 5
# of 8 with key pieces; the 8K layer.
@pytest.mark.parametrize("name,partition", [("tiny_d2", 0), ("gqa4_dh128_d4_r2", 1), ("split_keys_d8_r5", 0),
                                            ("llama7b_s8k_d8", 0)])
def test_c_caller_equals_binding(caller, name, partition, tmp_path):
    d, inp = _problem(name, partition)
    print(f"[case] C caller {name} partition={partition} {d}", flush=True)
    with open(tmp_path / "dims.txt", "w") as f:
        f.write(" ".join(str(v) for v in d.astuple()) + "\n")
    np.ascontiguousarray(inp["x"]).view(np.uint16).tofile(tmp_path / "x.bin")
    for k, v in pack_weights(inp, d).items():
        v.cpu().numpy().tofile(tmp_path / f"{k}.bin")
    rc = caller.tsp_c_caller_run(str(tmp_path).encode())
    assert rc == 0, "the C caller failed (its message is on stderr)"
    T = d.seq // d.degree
    y_c = np.fromfile(tmp_path / "y.bin", dtype=np.float32).reshape(d.batch, T, d.hidden)
    prob = RankProblem.build(d, inp)
    y = prob.layer().cpu().numpy()
    assert np.array_equal(y_c, y)
