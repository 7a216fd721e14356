"""CPU-only checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import synth
from folded_tensor_sequence_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tsp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        from folded_tensor_sequence_amd import build
        build.build()
    return B.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("tsp_zigzag_index", "tsp_qkv_proj", "tsp_kv_reorder", "tsp_attn_fwd",
              "tsp_mlp_ring_fwd", "tsp_layer_fwd", "tsp_workspace_bytes", "tsp_last_error",
              "tsp_profile_kernel", "tsp_profile_result"):
        assert n in names
    assert set(names) == set(B.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (tsp_\w+)", out))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def _dims(**kw):
    base = dict(batch=1, seq=256, degree=2, rank=0, hidden=256, n_q_heads=4, n_kv_heads=4,
                head_dim=64, ffn=768)
    base.update(kw)
    return B.TspDims(*base.values())


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)


@pytest.mark.parametrize("kw,code,frag", [
    (dict(batch=0), B.TSP_ERR_INVALID_ARG, "batch"),
    (dict(degree=0), B.TSP_ERR_INVALID_ARG, "degree"),
    (dict(rank=2), B.TSP_ERR_INVALID_ARG, "rank"),
    (dict(rank=-1), B.TSP_ERR_INVALID_ARG, "rank"),
    (dict(seq=250), B.TSP_ERR_INVALID_ARG, "seq"),
    (dict(seq=2), B.TSP_ERR_INVALID_ARG, "seq"),
    (dict(n_q_heads=3), B.TSP_ERR_INVALID_ARG, "multiples of degree"),
    (dict(n_kv_heads=6, n_q_heads=4), B.TSP_ERR_INVALID_ARG, "multiple of n_kv_heads"),
    (dict(hidden=200), B.TSP_ERR_INVALID_ARG, "hidden"),
    (dict(ffn=100), B.TSP_ERR_INVALID_ARG, "ffn"),
    (dict(ffn=64, degree=16, n_q_heads=16, n_kv_heads=16), B.TSP_ERR_INVALID_ARG, "ffn"),  # F/D = 4
    (dict(ffn=128, degree=3, seq=258, n_q_heads=6, n_kv_heads=3), B.TSP_ERR_INVALID_ARG, "ffn"),
    (dict(head_dim=96), B.TSP_ERR_UNSUPPORTED, "head_dim"),
    (dict(partition=2), B.TSP_ERR_INVALID_ARG, "partition"),
    (dict(partition=-1), B.TSP_ERR_INVALID_ARG, "partition"),
])
def test_invalid_dims_rejected(lib, kw, code, frag):
    d = _dims(**kw)
    rc = lib.tsp_layer_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           1 << 40, None)
    assert rc == code
    assert frag in lib.tsp_last_error().decode()
    assert lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_LAYER) == 0


def test_valid_edge_dims_accepted(lib):
    # F/D = 96 is not a multiple of 64 (ragged K segments) but is allowed; D = 1; c = 1
    for kw in (dict(ffn=192), dict(degree=1, rank=0), dict(seq=4, degree=2, rank=1)):
        assert lib.tsp_workspace_bytes(ctypes.byref(_dims(**kw)), B.TSP_FN_LAYER) > 0


def test_null_dims(lib):
    assert lib.tsp_zigzag_index(None, FAKE, None, None) == B.TSP_ERR_INVALID_ARG
    assert "dims" in lib.tsp_last_error().decode()


def test_null_and_misaligned_pointers(lib):
    d = _dims()
    big = 1 << 40
    rc = lib.tsp_layer_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "x_local is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_layer_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE,
                           big, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "w_down is not 16-byte aligned" in lib.tsp_last_error().decode()
    rc = lib.tsp_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, big, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "out is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None, big, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "ws is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_qkv_proj(ctypes.byref(d), 2, FAKE, FAKE, None, FAKE, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "src_rank" in lib.tsp_last_error().decode()
    rc = lib.tsp_qkv_proj(ctypes.byref(d), 1, FAKE, FAKE, MISALIGNED, FAKE, None)
    assert rc == B.TSP_ERR_INVALID_ARG and "q_out" in lib.tsp_last_error().decode()
    rc = lib.tsp_kv_reorder(ctypes.byref(d), FAKE, None, None)
    assert rc == B.TSP_ERR_INVALID_ARG
    rc = lib.tsp_zigzag_index(ctypes.byref(d), None, None, None)
    assert rc == B.TSP_ERR_INVALID_ARG


def test_workspace_too_small(lib):
    d = _dims()
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_LAYER)
    rc = lib.tsp_layer_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           need - 1, None)
    assert rc == B.TSP_ERR_WORKSPACE
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN)
    assert lib.tsp_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        B.TSP_ERR_WORKSPACE
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_MLP)
    assert lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, None) == \
        B.TSP_ERR_WORKSPACE
    assert lib.tsp_workspace_bytes(ctypes.byref(d), 99) == 0


def test_profile_arguments(lib):
    assert lib.tsp_profile_kernel(99, 1) == B.TSP_ERR_INVALID_ARG
    assert lib.tsp_profile_kernel(0, 0) == B.TSP_OK          # disarm is always fine
    assert lib.tsp_profile_result(None, None) == B.TSP_ERR_INVALID_ARG


def test_no_device_gives_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _dims()
    rc = lib.tsp_zigzag_index(ctypes.byref(d), FAKE, None, None)
    assert rc == B.TSP_ERR_HIP
    assert "HIP error" in lib.tsp_last_error().decode()


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workspace_sizes_match_layout(lib, name):
    # Exact sizes of the plain buffers; the workspaces must hold at least their
    # fixed pieces (the scratch for partial results depends on the work plan).
    d = synth.WORKLOADS[name].dims
    s = B.dims_struct(d)
    T = d.seq // d.degree
    M = d.batch * T
    c = d.seq // (2 * d.degree)
    kmax = (2 * d.degree - d.rank) * c
    kpad = -(-kmax // 64) * 64
    up = lambda x: -(-x // 256) * 256
    q = M * d.n_q_heads * d.head_dim * 2
    kvn = 2 * d.n_kv_heads * d.batch * kpad * d.head_dim * 2
    ws = lambda fn: lib.tsp_workspace_bytes(ctypes.byref(s), fn)
    assert ws(B.TSP_FN_KV_NATURAL) == kvn
    assert ws(B.TSP_FN_KV_GATHERED) == \
        d.degree * d.degree * 2 * d.batch * T * (d.n_kv_heads // d.degree) * d.head_dim * 2
    attn, mlp, layer = ws(B.TSP_FN_ATTN), ws(B.TSP_FN_MLP), ws(B.TSP_FN_LAYER)
    # attention reads K/V from the gathered buffer: its workspace is q and o
    fixed_attn = up(q) + up(q)
    fixed_mlp = up(M * d.hidden * 2) + up(M * d.ffn * 2)
    assert attn >= fixed_attn and mlp >= fixed_mlp
    scratch = attn - fixed_attn
    assert mlp - fixed_mlp <= scratch          # one scratch region sized for both
    assert layer == fixed_attn + up(M * d.hidden * 4) + fixed_mlp + scratch
    assert all(x % 256 == 0 for x in (attn, mlp, layer))


# The natural-order K/V buffer covers keys [0, kmax): one past the largest
# position any of the rank's rows attends to, which the oracle's partition
# maps give independently (zigzag (2D - r) c, striped (T - 1) D + r + 1).
@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
@pytest.mark.parametrize("S,D,r", [(256, 2, 0), (256, 2, 1), (384, 3, 2), (8192, 8, 0), (8192, 8, 7), (16, 8, 5)])
def test_kv_natural_size_follows_the_partition(lib, partition, S, D, r):
    from oracle import tsp_oracle as orc
    d = _dims(seq=S, degree=D, rank=r, n_q_heads=2 * D, n_kv_heads=D, ffn=64 * D, partition=partition)
    kmax = int(orc.local_to_global(S, D, r, partition).max()) + 1
    kpad = -(-kmax // 64) * 64
    want = 2 * D * 1 * kpad * 64 * 2   # K and V, Hkv heads, B = 1, dh = 64, 2 bytes
    assert lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_KV_NATURAL) == want


def test_dims_struct_carries_the_partition():
    names = [f[0] for f in B.TspDims._fields_]
    assert names[-1] == "partition" and len(names) == 10
    d = synth.Dims(1, 256, 2, 0, 256, 4, 4, 64, 768, partition=1)
    assert B.dims_struct(d).partition == 1
    assert B.dims_struct(synth.Dims(1, 256, 2, 0, 256, 4, 4, 64, 768)).partition == 0
