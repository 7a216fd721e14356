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
              "tsp_profile_kernel", "tsp_profile_result", "tsp_set_tuning"):
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
    (dict(batch=0), B.TSP_ERR_BATCH, "batch"),
    (dict(degree=0), B.TSP_ERR_DEGREE, "degree"),
    (dict(rank=2), B.TSP_ERR_RANK, "rank"),
    (dict(rank=-1), B.TSP_ERR_RANK, "rank"),
    (dict(seq=250), B.TSP_ERR_SEQ, "seq"),
    (dict(seq=2), B.TSP_ERR_SEQ, "seq"),
    (dict(n_q_heads=3), B.TSP_ERR_HEADS, "multiples of degree"),
    (dict(n_q_heads=0), B.TSP_ERR_HEADS, "head counts"),
    (dict(n_kv_heads=6, n_q_heads=4), B.TSP_ERR_GQA, "multiple of n_kv_heads"),
    (dict(hidden=200), B.TSP_ERR_HIDDEN, "hidden"),
    (dict(ffn=100), B.TSP_ERR_FFN, "ffn"),
    (dict(ffn=64, degree=16, n_q_heads=16, n_kv_heads=16), B.TSP_ERR_FFN, "ffn"),  # F/D = 4
    (dict(ffn=128, degree=3, seq=258, n_q_heads=6, n_kv_heads=3), B.TSP_ERR_FFN, "ffn"),
    (dict(head_dim=96), B.TSP_ERR_UNSUPPORTED, "head_dim"),
    (dict(partition=2), B.TSP_ERR_PARTITION, "partition"),
    (dict(partition=-1), B.TSP_ERR_PARTITION, "partition"),
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
    assert lib.tsp_zigzag_index(None, FAKE, None, None) == B.TSP_ERR_NULL_POINTER
    assert "dims" in lib.tsp_last_error().decode()


def test_error_codes_are_distinct():
    codes = {k: v for k, v in vars(B).items() if k.startswith("TSP_ERR_")}
    assert len(set(codes.values())) == len(codes)
    # the header declares the same set with the same values
    text = open(HEADER).read()
    declared = dict((n, int(v)) for n, v in re.findall(r"\b(TSP_ERR_\w+)\s*=\s*(-?\d+)", text))
    assert declared == codes


def test_null_and_misaligned_pointers(lib):
    d = _dims()
    big = 1 << 40
    rc = lib.tsp_layer_fwd(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, big, None)
    assert rc == B.TSP_ERR_NULL_POINTER and "x_local is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_layer_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, FAKE,
                           big, None)
    assert rc == B.TSP_ERR_MISALIGNED and "w_down is not 16-byte aligned" in lib.tsp_last_error().decode()
    rc = lib.tsp_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, None, FAKE, big, None)
    assert rc == B.TSP_ERR_NULL_POINTER and "out is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, big, None)
    assert rc == B.TSP_ERR_MISALIGNED and "residual" in lib.tsp_last_error().decode()
    rc = lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, B.TSP_F32, FAKE, FAKE, FAKE, None, FAKE, None, big, None)
    assert rc == B.TSP_ERR_NULL_POINTER and "ws is NULL" in lib.tsp_last_error().decode()
    rc = lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, B.TSP_F32, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE, big, None)
    assert rc == B.TSP_ERR_MISALIGNED and "residual" in lib.tsp_last_error().decode()
    for bad in (3, -1):
        rc = lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, bad, FAKE, FAKE, FAKE, None, FAKE, FAKE, big, None)
        assert rc == B.TSP_ERR_DTYPE and "x_dtype" in lib.tsp_last_error().decode()
    rc = lib.tsp_qkv_proj(ctypes.byref(d), 2, FAKE, FAKE, None, FAKE, None)
    assert rc == B.TSP_ERR_RANK and "src_rank" in lib.tsp_last_error().decode()
    rc = lib.tsp_qkv_proj(ctypes.byref(d), 1, FAKE, FAKE, MISALIGNED, FAKE, None)
    assert rc == B.TSP_ERR_MISALIGNED and "q_out" in lib.tsp_last_error().decode()
    rc = lib.tsp_kv_reorder(ctypes.byref(d), FAKE, None, 0, None)
    assert rc == B.TSP_ERR_NULL_POINTER
    for bad in (-1, 257):
        rc = lib.tsp_kv_reorder(ctypes.byref(d), FAKE, FAKE, bad, None)
        assert rc == B.TSP_ERR_KMAX and "kmax" in lib.tsp_last_error().decode()
    rc = lib.tsp_zigzag_index(ctypes.byref(d), None, None, None)
    assert rc == B.TSP_ERR_NULL_POINTER


def test_workspace_too_small(lib):
    d = _dims()
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_LAYER)
    rc = lib.tsp_layer_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           need - 1, None)
    assert rc == B.TSP_ERR_WORKSPACE
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN)
    assert lib.tsp_attn_fwd(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, need - 1, None) == \
        B.TSP_ERR_WORKSPACE
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_MLP)
    assert lib.tsp_mlp_ring_fwd(ctypes.byref(d), FAKE, B.TSP_BF16, FAKE, FAKE, FAKE, None, FAKE, FAKE, need - 1,
                                None) == B.TSP_ERR_WORKSPACE
    assert lib.tsp_workspace_bytes(ctypes.byref(d), 99) == 0


def test_tuning_knobs(lib):
    assert lib.tsp_set_tuning(B.TUNE["attn_pair"], 0) == B.TSP_OK
    assert lib.tsp_set_tuning(B.TUNE["attn_pair"], -1) == B.TSP_OK
    assert lib.tsp_set_tuning(99, 1) == B.TSP_ERR_INVALID_ARG
    assert lib.tsp_set_tuning(-1, 1) == B.TSP_ERR_INVALID_ARG
    # the header's knob list matches the binding's
    text = open(HEADER).read()
    declared = dict((n, int(v)) for n, v in re.findall(r"\bTSP_TUNE_(\w+)\s*=\s*(\d+)", text))
    assert {k.lower(): v for k, v in declared.items() if k != "COUNT"} == B.TUNE


def test_profile_arguments(lib):
    assert lib.tsp_profile_kernel(99, 1) == B.TSP_ERR_INVALID_ARG
    assert lib.tsp_profile_kernel(0, 0) == B.TSP_OK          # disarm is always fine
    assert lib.tsp_profile_result(None, None) == B.TSP_ERR_NULL_POINTER


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


# --------------------------------------------------------------------------- #
# The binding rejects tensors that do not fit the ABI before calling the library
# --------------------------------------------------------------------------- #
def _tiny():
    return synth.WORKLOADS["tiny_d2"].dims


def test_binding_rejects_host_tensors():
    import torch
    d = _tiny()
    T = d.seq // d.degree
    x = torch.zeros((d.batch, T, d.hidden), dtype=torch.int16)        # on the host
    with pytest.raises(ValueError, match="GPU tensor"):
        B.tsp_qkv_proj(d, 0, x, x, None, x)
    l2g = torch.zeros(T, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        B.tsp_zigzag_index(d, l2g)


class _FakeCuda:
    """Stands in for a GPU tensor on a machine without one (only the fields the
    binding's checks read); its pointer is never used because every case below
    fails a check first."""

    def __init__(self, n, dtype, contiguous=True):
        import torch
        self._t = torch.empty(n, dtype=dtype)
        self.dtype = dtype
        self._contig = contiguous
        self.is_cuda = True
        self.device = "cuda:0"

    def is_contiguous(self):
        return self._contig

    def numel(self):
        return self._t.numel()

    def element_size(self):
        return self._t.element_size()


@pytest.mark.parametrize("case", ["dtype", "short", "noncontig", "notensor"])
def test_binding_checks_dtype_size_layout(case, monkeypatch):
    import torch
    monkeypatch.setattr(torch, "Tensor", _FakeCuda)       # isinstance() accepts the fake
    d = _tiny()
    z = B._Sizes(d)
    if case == "dtype":
        t, msg = _FakeCuda(z.rows, torch.float32), "must be bf16"
    elif case == "short":
        t, msg = _FakeCuda(z.rows - 1, torch.int16), "bytes, the ABI layout needs"
    elif case == "noncontig":
        t, msg = _FakeCuda(z.rows, torch.int16, contiguous=False), "contiguous"
    else:
        t, msg = object(), "torch.Tensor"
    with pytest.raises(ValueError, match=msg):
        B._tensor(t, "x_local", "bf16", z.x16)


def test_binding_sizes_follow_the_header():
    d = synth.WORKLOADS["llama7b_s8k_d8"].dims
    z = B._Sizes(d)
    assert z.x16 == 1024 * 4096 * 2 and z.f32 == 1024 * 4096 * 4
    assert z.w_qkv == 2 * 96 * 128 * 4096 and z.w_o == 2 * 4096 * 4096 and z.w_ffn == 2 * 11008 * 4096
    assert z.q == 2 * 1024 * 32 * 128
    # default kmax of rank 0 = (2D - r) c = 16 * 512; natural K and V, 32 heads
    assert z.kv_natural(0) == 4 * 32 * 8192 * 128
    assert z.kv_natural(100) == 4 * 32 * 128 * 128


def test_noalloc_rejects_layers_beyond_the_scratch_array(lib):
    text = open(HEADER).read()
    m = re.search(r"#define TSP_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)", text)
    assert m and int(m.group(1)) * 1024 * 1024 == B.TSP_SCRATCH_BYTES
    big = B.dims_struct(synth.WORKLOADS["llama3_8b_gqa_s16k_d8"].dims)
    assert lib.tsp_workspace_bytes(ctypes.byref(big), B.TSP_FN_LAYER) > B.TSP_SCRATCH_BYTES
    rc = lib.tsp_layer_fwd_noalloc(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == B.TSP_ERR_SCRATCH and "scratch array" in lib.tsp_last_error().decode()
    # the headline layer fits
    l7 = B.dims_struct(synth.WORKLOADS["llama7b_s8k_d8"].dims)
    assert lib.tsp_workspace_bytes(ctypes.byref(l7), B.TSP_FN_LAYER) <= B.TSP_SCRATCH_BYTES
    # argument checks come first
    rc = lib.tsp_layer_fwd_noalloc(ctypes.byref(l7), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None)
    assert rc == B.TSP_ERR_NULL_POINTER and "y is NULL" in lib.tsp_last_error().decode()


def test_noalloc_without_device_gives_hip_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    d = _dims()
    rc = lib.tsp_layer_fwd_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == B.TSP_ERR_HIP


def test_mlp_bwd_argument_checks(lib):
    d = _dims()
    big = 1 << 40
    f = lib.tsp_mlp_ring_bwd
    args = lambda **kw: [kw.get(n, FAKE) for n in ("x",)] + [kw.get("xdt", B.TSP_BF16)] + \
        [kw.get(n, FAKE) for n in ("dy", "wg", "wu", "wd")] + [kw.get("res", None)] + \
        [kw.get(n, FAKE) for n in ("dx", "dwg", "dwu", "dwd", "ws")]
    assert f(ctypes.byref(d), *args(xdt=7), big, None) == B.TSP_ERR_DTYPE
    assert f(ctypes.byref(d), *args(dy=None), big, None) == B.TSP_ERR_NULL_POINTER
    assert "dy is NULL" in lib.tsp_last_error().decode()
    assert f(ctypes.byref(d), *args(dwd=None), big, None) == B.TSP_ERR_NULL_POINTER
    assert f(ctypes.byref(d), *args(res=MISALIGNED), big, None) == B.TSP_ERR_MISALIGNED
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_MLP_BWD)
    assert need > 0 and need % 256 == 0
    assert f(ctypes.byref(d), *args(), need - 1, None) == B.TSP_ERR_WORKSPACE
    bad = _dims(batch=0)
    assert f(ctypes.byref(bad), *args(), big, None) == B.TSP_ERR_BATCH


def test_attn_bwd_argument_checks(lib):
    d = _dims()
    big = 1 << 40
    f = lib.tsp_attn_bwd
    names = ("x", "wqkv", "wo", "kv", "dh", "dq", "send", "dwo", "ws")
    args = lambda **kw: [kw.get(n, FAKE) for n in names]
    for n, label in zip(names, ("x_local", "w_qkv", "w_o", "kv_gathered", "dh", "dq", "dkv_send", "dw_o", "ws")):
        assert f(ctypes.byref(d), *args(**{n: None}), big, None) == B.TSP_ERR_NULL_POINTER
        assert f"{label} is NULL" in lib.tsp_last_error().decode()
    assert f(ctypes.byref(d), *args(dh=MISALIGNED), big, None) == B.TSP_ERR_MISALIGNED
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN_BWD)
    assert need > 0 and need % 256 == 0
    assert f(ctypes.byref(d), *args(), need - 1, None) == B.TSP_ERR_WORKSPACE
    assert f(ctypes.byref(_dims(rank=5)), *args(), big, None) == B.TSP_ERR_RANK
    g = lib.tsp_attn_bwd_proj
    pnames = ("x", "wqkv", "dq", "own", "res", "dx", "dwqkv", "ws")
    pargs = lambda **kw: [kw.get(n, None if n == "res" else FAKE) for n in pnames]
    assert g(ctypes.byref(d), *pargs(own=None), big, None) == B.TSP_ERR_NULL_POINTER
    assert "dkv_own is NULL" in lib.tsp_last_error().decode()
    assert g(ctypes.byref(d), *pargs(res=MISALIGNED), big, None) == B.TSP_ERR_MISALIGNED
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN_BWD_PROJ)
    assert g(ctypes.byref(d), *pargs(), need - 1, None) == B.TSP_ERR_WORKSPACE
    # past validation, no device: a HIP error, nothing launched
    if not __import__("torch").cuda.is_available():
        assert g(ctypes.byref(d), *pargs(), big, None) == B.TSP_ERR_HIP


@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_attn_bwd_buffer_sizes(lib, name):
    # the K/V-gradient send buffer: [D dst][D shard][K|V][B][T][Hkv/D dh] float32
    d = synth.WORKLOADS[name].dims
    s = B.dims_struct(d)
    T = d.seq // d.degree
    assert lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_DKV) == \
        d.degree * d.degree * 2 * d.batch * T * (d.n_kv_heads // d.degree) * d.head_dim * 4
    for fn in (B.TSP_FN_ATTN_BWD, B.TSP_FN_ATTN_BWD_PROJ):
        n = lib.tsp_workspace_bytes(ctypes.byref(s), fn)
        assert n > 0 and n % 256 == 0


def _up256(n):
    return (n + 255) // 256 * 256


@pytest.mark.parametrize("name", ["llama7b_s8k_d8", "tiny_d2"])
def test_bwd_weight_copies_in_workspace(lib, name):
    # The backward calls read W_down, W_gate/W_up, W_O and W_QKV as stored;
    # TSP_TUNE_BWD_WEIGHTS = 1 switches to transposed copies, which the
    # workspaces then hold: exactly one extra weight-sized piece per copy.
    d = synth.WORKLOADS[name].dims
    s = B.dims_struct(d)
    h, F, qd = d.hidden, d.ffn, d.n_q_heads * d.head_dim
    nall = (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim
    fns = (B.TSP_FN_MLP_BWD, B.TSP_FN_ATTN_BWD, B.TSP_FN_ATTN_BWD_PROJ)
    assert (F // d.degree) % 32 == 0  # the K-major dx applies to both shapes
    base = [lib.tsp_workspace_bytes(ctypes.byref(s), fn) for fn in fns]
    try:
        assert lib.tsp_set_tuning(B.TUNE["bwd_weights"], 1) == B.TSP_OK
        copies = [lib.tsp_workspace_bytes(ctypes.byref(s), fn) for fn in fns]
    finally:
        lib.tsp_set_tuning(B.TUNE["bwd_weights"], -1)
    assert copies[0] - base[0] == _up256(F * h * 2) + _up256(2 * F * h * 2)
    assert copies[1] - base[1] == _up256(qd * h * 2)
    assert copies[2] - base[2] == _up256(nall * h * 2)
    assert [lib.tsp_workspace_bytes(ctypes.byref(s), fn) for fn in fns] == base


def test_bwd_dx_copies_when_shard_width_is_not_a_multiple_of_32(lib):
    # F/D = 176: the K-major dx of the MLP backward does not apply (its K
    # segments of 2 F/D are not whole multiples of 64), so the workspace
    # holds the transposed W_gate / W_up copy whatever the knob says
    d = synth.Dims(1, 256, 4, 3, 192, 8, 4, 64, 704, 0)
    s = B.dims_struct(d)
    base = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_MLP_BWD)
    try:
        assert lib.tsp_set_tuning(B.TUNE["bwd_weights"], 1) == B.TSP_OK
        copies = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_MLP_BWD)
    finally:
        lib.tsp_set_tuning(B.TUNE["bwd_weights"], -1)
    assert copies - base == _up256(704 * 192 * 2)


def test_attn_keep_argument_checks_and_sizes(lib):
    d = _dims()
    s = B.dims_struct(synth.WORKLOADS["llama7b_s8k_d8"].dims)
    big = 1 << 40
    # kept tensors: lse is float32 [B][Hq][T]; the kept backward's workspace is
    # the recomputing one without q, o and lse
    wl = synth.WORKLOADS["llama7b_s8k_d8"].dims
    T = wl.seq // wl.degree
    rows = wl.batch * wl.n_q_heads * T
    assert lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_LSE) == rows * 4
    qo = wl.batch * T * wl.n_q_heads * wl.head_dim * 2
    full = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_ATTN_BWD)
    kept = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_ATTN_BWD_KEPT)
    assert full - kept == 2 * _up256(qo) + _up256(rows * 4)
    assert lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_ATTN_KEEP) > 0
    f = lib.tsp_attn_fwd_keep
    names = ("x", "wqkv", "wo", "kv", "res", "out", "q", "o", "lse", "ws")
    args = lambda **kw: [kw.get(n, None if n == "res" else FAKE) for n in names]
    for n, label in (("q", "q_keep"), ("o", "o_keep"), ("lse", "lse_keep"), ("out", "out")):
        assert f(ctypes.byref(d), *args(**{n: None}), big, None) == B.TSP_ERR_NULL_POINTER
        assert f"{label} is NULL" in lib.tsp_last_error().decode()
    assert f(ctypes.byref(d), *args(lse=MISALIGNED), big, None) == B.TSP_ERR_MISALIGNED
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN_KEEP)
    assert f(ctypes.byref(d), *args(), need - 1, None) == B.TSP_ERR_WORKSPACE
    g = lib.tsp_attn_bwd_kept
    gnames = ("wo", "kv", "q", "o", "lse", "dh", "dq", "send", "dwo", "ws")
    gargs = lambda **kw: [kw.get(n, FAKE) for n in gnames]
    for n, label in zip(gnames, ("w_o", "kv_gathered", "q_keep", "o_keep", "lse_keep", "dh", "dq", "dkv_send",
                                 "dw_o", "ws")):
        assert g(ctypes.byref(d), *gargs(**{n: None}), big, None) == B.TSP_ERR_NULL_POINTER
        assert f"{label} is NULL" in lib.tsp_last_error().decode()
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_ATTN_BWD_KEPT)
    assert g(ctypes.byref(d), *gargs(), need - 1, None) == B.TSP_ERR_WORKSPACE
    assert g(ctypes.byref(_dims(rank=5)), *gargs(), big, None) == B.TSP_ERR_RANK


def test_mlp_keep_argument_checks_and_sizes(lib):
    d = _dims()
    big = 1 << 40
    # kept tensor: g then u, float32 [2][B][T][F]; the kept backward's
    # workspace is the recomputing one without dA and the f16 copy of x
    wl = synth.WORKLOADS["llama7b_s8k_d8"].dims
    s = B.dims_struct(wl)
    M = wl.batch * (wl.seq // wl.degree)
    assert lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_GU) == 2 * M * wl.ffn * 4
    full = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_MLP_BWD)
    kept = lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_MLP_BWD_KEPT)
    assert full - kept == _up256(M * wl.hidden * 2) + _up256(M * wl.ffn * 4)
    f = lib.tsp_mlp_ring_fwd_keep
    names = ("x", "wg", "wu", "wd", "res", "y", "gu", "ws")
    args = lambda **kw: [kw.get(n, None if n == "res" else FAKE) for n in names]
    call = lambda xdt=B.TSP_BF16, nbytes=big, **kw: f(ctypes.byref(d), *args(**kw)[:1], xdt, *args(**kw)[1:],
                                                      nbytes, None)
    for n, label in (("gu", "gu_keep"), ("y", "y"), ("x", "x"), ("ws", "ws")):
        assert call(**{n: None}) == B.TSP_ERR_NULL_POINTER
        assert f"{label} is NULL" in lib.tsp_last_error().decode()
    assert call(gu=MISALIGNED) == B.TSP_ERR_MISALIGNED
    assert call(xdt=7) == B.TSP_ERR_DTYPE
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_MLP)
    assert call(nbytes=need - 1) == B.TSP_ERR_WORKSPACE
    g = lib.tsp_mlp_ring_bwd_kept
    gnames = ("x", "dy", "wg", "wu", "wd", "gu", "dxr", "dx", "dwg", "dwu", "dwd", "ws")
    gargs = lambda **kw: [kw.get(n, None if n == "dxr" else FAKE) for n in gnames]
    gcall = lambda nbytes=big, rank_dims=d, **kw: g(ctypes.byref(rank_dims), *gargs(**kw)[:1], B.TSP_BF16,
                                                    *gargs(**kw)[1:], nbytes, None)
    for n, label in zip(gnames, ("x", "dy", "w_gate", "w_up", "w_down", "gu_keep", None, "dx", "dw_gate", "dw_up",
                                 "dw_down", "ws")):
        if label is None:
            continue
        assert gcall(**{n: None}) == B.TSP_ERR_NULL_POINTER
        assert f"{label} is NULL" in lib.tsp_last_error().decode()
    need = lib.tsp_workspace_bytes(ctypes.byref(d), B.TSP_FN_MLP_BWD_KEPT)
    assert gcall(nbytes=need - 1) == B.TSP_ERR_WORKSPACE
    assert gcall(rank_dims=_dims(rank=5)) == B.TSP_ERR_RANK


@pytest.mark.parametrize("name", ["llama7b_s8k_d8", "llama3_8b_gqa_s16k_d8", "tiny_d2"])
def test_kept_bytes_match_the_memory_calculator(lib, name):
    # the calculator's count of what the kept-activation calls hold per rank
    # and layer (written from the shapes) against the library's buffer sizes
    from folded_tensor_sequence_amd import memory_model as mm
    d = synth.WORKLOADS[name].dims
    s = B.dims_struct(d)
    model = mm.Model(params=0.0, hidden=d.hidden, layers=1, n_q_heads=d.n_q_heads, n_kv_heads=d.n_kv_heads,
                     head_dim=d.head_dim, ffn=d.ffn)
    kept = mm.kept_activation_bytes(model, d.seq, d.batch, d.degree)
    qo = 2 * B._Sizes(d).q
    assert kept["attention"] == qo + lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_LSE)
    assert kept["mlp"] == lib.tsp_workspace_bytes(ctypes.byref(s), B.TSP_FN_GU)
