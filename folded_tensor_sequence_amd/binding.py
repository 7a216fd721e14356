"""ctypes binding of libtsp.so: same names as the C ABI, argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI; this module
turns torch tensors into device pointers and the current HIP stream into a
``hipStream_t``.  If the library is not built it raises -- there is no CPU
fallback.

Before a pointer is handed over, each wrapper checks that the tensor lives on
a GPU, is contiguous, has an element type of the width the ABI expects, and
holds at least the bytes the ABI layout implies for these dims; a mismatch
raises ``ValueError`` and nothing reaches the library.  16-bit tensors may be
``int16`` / ``uint16`` bit patterns or the matching float type.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtsp.so")

TSP_OK = 0
TSP_ERR_INVALID_ARG = -1
TSP_ERR_UNSUPPORTED = -2
TSP_ERR_WORKSPACE = -3
TSP_ERR_HIP = -4
TSP_ERR_NULL_POINTER = -5
TSP_ERR_MISALIGNED = -6
TSP_ERR_BATCH = -10
TSP_ERR_DEGREE = -11
TSP_ERR_RANK = -12
TSP_ERR_SEQ = -13
TSP_ERR_HEADS = -14
TSP_ERR_GQA = -15
TSP_ERR_HIDDEN = -16
TSP_ERR_FFN = -17
TSP_ERR_PARTITION = -18
TSP_ERR_DTYPE = -19
TSP_ERR_KMAX = -20
TSP_ERR_SCRATCH = -21

TSP_BF16, TSP_F16, TSP_F32 = 0, 1, 2

TSP_FN_ATTN = 1
TSP_FN_MLP = 2
TSP_FN_LAYER = 3
TSP_FN_KV_NATURAL = 4
TSP_FN_KV_GATHERED = 5
TSP_FN_MLP_BWD = 6
TSP_FN_ATTN_BWD = 7
TSP_FN_ATTN_BWD_PROJ = 8
TSP_FN_DKV = 9
TSP_FN_ATTN_KEEP = 10
TSP_FN_ATTN_BWD_KEPT = 11
TSP_FN_LSE = 12
TSP_FN_MLP_BWD_KEPT = 13
TSP_FN_GU = 14

KERNELS = {"qkv": 1, "reorder": 2, "attn": 3, "oproj": 4, "gateup": 5, "down": 6, "attn_bwd": 7}

TUNE = {"gemm_qkv": 0, "gemm_oproj": 1, "gemm_gateup": 2, "gemm_down": 3, "split_oproj": 4,
        "split_down": 5, "attn_shape": 6, "attn_pair": 7, "attn_pieces": 8, "bwd_weights": 9}

EXPORTED = ("tsp_zigzag_index", "tsp_qkv_proj", "tsp_kv_reorder", "tsp_attn_fwd",
            "tsp_mlp_ring_fwd", "tsp_layer_fwd", "tsp_workspace_bytes", "tsp_last_error",
            "tsp_profile_kernel", "tsp_profile_result", "tsp_set_tuning", "tsp_layer_fwd_noalloc",
            "tsp_mlp_ring_bwd", "tsp_attn_bwd", "tsp_attn_bwd_proj", "tsp_attn_fwd_keep",
            "tsp_attn_bwd_kept", "tsp_mlp_ring_fwd_keep", "tsp_mlp_ring_bwd_kept")

# Size of the library's fixed scratch array (TSP_SCRATCH_BYTES in include/tsp.h).
TSP_SCRATCH_BYTES = 128 * 1024 * 1024


class TspDims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "seq", "degree", "rank", "hidden",
                                               "n_q_heads", "n_kv_heads", "head_dim", "ffn",
                                               "partition")]


class TspError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libtsp error {code}: {msg}")
        self.code = code


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libtsp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(folded_tensor_sequence_amd/build.py); there is no fallback path")
    lib = ctypes.CDLL(path)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    dp = ctypes.POINTER(TspDims)
    sig = {
        "tsp_zigzag_index": [dp, vp, vp, vp],
        "tsp_qkv_proj": [dp, i32, vp, vp, vp, vp, vp],
        "tsp_kv_reorder": [dp, vp, vp, i32, vp],
        "tsp_attn_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_mlp_ring_fwd": [dp, vp, i32, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_layer_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_layer_fwd_noalloc": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "tsp_mlp_ring_bwd": [dp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_attn_bwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_attn_bwd_proj": [dp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_attn_fwd_keep": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_attn_bwd_kept": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_mlp_ring_fwd_keep": [dp, vp, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_mlp_ring_bwd_kept": [dp, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.tsp_workspace_bytes.argtypes = [dp, i32]
    lib.tsp_workspace_bytes.restype = sz
    lib.tsp_profile_kernel.argtypes = [i32, i32]
    lib.tsp_profile_kernel.restype = ctypes.c_int
    lib.tsp_profile_result.argtypes = [ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_float)]
    lib.tsp_profile_result.restype = ctypes.c_int
    lib.tsp_set_tuning.argtypes = [i32, i32]
    lib.tsp_set_tuning.restype = ctypes.c_int
    lib.tsp_last_error.argtypes = []
    lib.tsp_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def dims_struct(dims) -> TspDims:
    if isinstance(dims, TspDims):
        return dims
    return TspDims(dims.batch, dims.seq, dims.degree, dims.rank, dims.hidden,
                   dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.ffn,
                   getattr(dims, "partition", 0))


# --------------------------------------------------------------------------- #
# Argument checks (host side, before any pointer reaches the library)
# --------------------------------------------------------------------------- #
_KINDS = {
    "bf16": (torch.int16, torch.uint16, torch.bfloat16),
    "f16": (torch.int16, torch.uint16, torch.float16),
    "f32": (torch.float32,),
    "i32": (torch.int32,),
    "bytes": None,  # any element type (workspace)
}


def _tensor(t, name: str, kind: str, nbytes: int | None, optional: bool = False):
    """Device pointer of ``t`` after checking device, layout, type and size."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor (got {type(t).__name__})")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (got device {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    allowed = _KINDS[kind]
    if allowed is not None and t.dtype not in allowed:
        raise ValueError(f"{name} must be {kind} ({', '.join(str(a) for a in allowed)}), got {t.dtype}")
    have = t.numel() * t.element_size()
    if nbytes is not None and have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the ABI layout needs {nbytes}")
    return ctypes.c_void_p(t.data_ptr())


class _Sizes:
    """Byte sizes of the ABI layouts for one dims (include/tsp.h)."""

    def __init__(self, dims):
        d = dims
        self.T = d.seq // d.degree
        self.M = d.batch * self.T
        self.rows = self.M * d.hidden                         # [B][T][h]
        self.x16 = 2 * self.rows
        self.f32 = 4 * self.rows
        self.w_qkv = 2 * (d.n_q_heads + 2 * d.n_kv_heads) * d.head_dim * d.hidden
        self.w_o = 2 * d.hidden * d.n_q_heads * d.head_dim
        self.w_ffn = 2 * d.ffn * d.hidden
        self.q = 2 * self.M * d.n_q_heads * d.head_dim
        self.dq = 2 * self.q                                  # float32 [B][T][Hq*dh]
        self.dkv_own = 4 * 2 * self.M * d.n_kv_heads * d.head_dim
        self.l2g = 4 * self.T
        self.g2s = 4 * d.seq
        self.dims = d

    def kv_natural(self, kmax):
        d = self.dims
        if kmax == 0:
            c = d.seq // (2 * d.degree)
            kmax = ((self.T - 1) * d.degree + d.rank + 1 if getattr(d, "partition", 0) == 1
                    else (2 * d.degree - d.rank) * c)
        kpad = -(-kmax // 64) * 64
        return 4 * d.n_kv_heads * d.batch * kpad * d.head_dim


def _s(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(rc: int):
    if rc != TSP_OK:
        raise TspError(rc, load().tsp_last_error().decode())


def _nbytes(t):
    return t.numel() * t.element_size()


def tsp_workspace_bytes(dims, fn: int) -> int:
    d = dims_struct(dims)
    n = load().tsp_workspace_bytes(ctypes.byref(d), fn)
    if n == 0:
        raise TspError(TSP_ERR_INVALID_ARG, load().tsp_last_error().decode())
    return n


def _ws(dims, ws, fn):
    return _tensor(ws, "ws", "bytes", tsp_workspace_bytes(dims, fn)), _nbytes(ws)


def tsp_zigzag_index(dims, local_to_global, global_to_slot=None, stream=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    _check(load().tsp_zigzag_index(ctypes.byref(d), _tensor(local_to_global, "local_to_global", "i32", z.l2g),
                                   _tensor(global_to_slot, "global_to_slot", "i32", z.g2s, optional=True),
                                   _s(stream)))


def tsp_qkv_proj(dims, src_rank, x_shard, w_qkv, q_out, kv_gathered, stream=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    _check(load().tsp_qkv_proj(ctypes.byref(d), int(src_rank), _tensor(x_shard, "x_shard", "bf16", z.x16),
                               _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv),
                               _tensor(q_out, "q_out", "f16", z.q, optional=True),
                               _tensor(kv_gathered, "kv_gathered", "f16",
                                       tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
                               _s(stream)))


def tsp_kv_reorder(dims, kv_gathered, kv_natural, kmax: int = 0, stream=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    kmax = int(kmax)
    nat_bytes = z.kv_natural(kmax) if 0 <= kmax <= d.seq else None  # else the library says why
    _check(load().tsp_kv_reorder(ctypes.byref(d),
                                 _tensor(kv_gathered, "kv_gathered", "f16",
                                         tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
                                 _tensor(kv_natural, "kv_natural", "f16", nat_bytes), kmax, _s(stream)))


def tsp_attn_fwd(dims, x_local, w_qkv, w_o, kv_gathered, out, ws, residual=None, stream=None):
    """out = residual + attention branch (residual None: the branch alone)."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_ATTN)
    _check(load().tsp_attn_fwd(ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16),
                               _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv), _tensor(w_o, "w_o", "bf16", z.w_o),
                               _tensor(kv_gathered, "kv_gathered", "f16",
                                       tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
                               _tensor(residual, "residual", "f32", z.f32, optional=True),
                               _tensor(out, "out", "f32", z.f32), wsp, wsn, _s(stream)))


_XDTYPE = {torch.bfloat16: TSP_BF16, torch.float16: TSP_F16, torch.float32: TSP_F32}


def _x_kind(x, x_dtype):
    """(x_dtype, tensor kind) of an MLP input: x_dtype TSP_BF16 / TSP_F16 /
    TSP_F32, or None to take it from x's torch dtype (bfloat16, float16 or
    float32; 16-bit integer bit patterns need x_dtype)."""
    if x_dtype is None:
        if not isinstance(x, torch.Tensor) or x.dtype not in _XDTYPE:
            raise ValueError("x_dtype is required unless x is bfloat16, float16 or float32")
        x_dtype = _XDTYPE[x.dtype]
    kind = {TSP_BF16: "bf16", TSP_F16: "f16", TSP_F32: "f32"}.get(int(x_dtype))
    if kind is None:
        raise ValueError(f"x_dtype {x_dtype} unknown")
    return int(x_dtype), kind


def _mlp_fwd(fn, dims, x, w_gate, w_up, w_down, y, ws, residual, x_dtype, stream, gu_keep=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    x_dtype, kind = _x_kind(x, x_dtype)
    wsp, wsn = _ws(dims, ws, TSP_FN_MLP)
    head = [ctypes.byref(d), _tensor(x, "x", kind, z.f32 if kind == "f32" else z.x16), x_dtype,
            _tensor(w_gate, "w_gate", "bf16", z.w_ffn), _tensor(w_up, "w_up", "bf16", z.w_ffn),
            _tensor(w_down, "w_down", "bf16", z.w_ffn), _tensor(residual, "residual", "f32", z.f32, optional=True),
            _tensor(y, "y", "f32", z.f32)]
    if fn == "tsp_mlp_ring_fwd_keep":
        head.append(_tensor(gu_keep, "gu_keep", "f32", tsp_workspace_bytes(dims, TSP_FN_GU)))
    _check(getattr(load(), fn)(*head, wsp, wsn, _s(stream)))


def tsp_mlp_ring_fwd(dims, x, w_gate, w_up, w_down, y, ws, residual=None, x_dtype=None, stream=None):
    """y = residual + MLP ring over x (residual None: the MLP branch alone).

    x_dtype: TSP_BF16 / TSP_F16 / TSP_F32; None takes it from x's torch dtype
    (bfloat16, float16 or float32; 16-bit integer bit patterns need x_dtype)."""
    _mlp_fwd("tsp_mlp_ring_fwd", dims, x, w_gate, w_up, w_down, y, ws, residual, x_dtype, stream)


def tsp_mlp_ring_fwd_keep(dims, x, w_gate, w_up, w_down, y, gu_keep, ws, residual=None, x_dtype=None, stream=None):
    """tsp_mlp_ring_fwd that also hands g = x Wg^T and u = x Wu^T (float32
    [2][B][T][F]: g, then u) to the caller, for tsp_mlp_ring_bwd_kept."""
    _mlp_fwd("tsp_mlp_ring_fwd_keep", dims, x, w_gate, w_up, w_down, y, ws, residual, x_dtype, stream, gu_keep)


def _mlp_bwd(fn, dims, x, dy, w_gate, w_up, w_down, dx, dw_gate, dw_up, dw_down, ws, dx_residual, x_dtype, stream,
             gu_keep=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    x_dtype, kind = _x_kind(x, x_dtype)
    kept = fn == "tsp_mlp_ring_bwd_kept"
    wsp, wsn = _ws(dims, ws, TSP_FN_MLP_BWD_KEPT if kept else TSP_FN_MLP_BWD)
    fw = 2 * z.w_ffn      # float32 gradient of a [F][h] weight
    args = [ctypes.byref(d), _tensor(x, "x", kind, z.f32 if kind == "f32" else z.x16), x_dtype,
            _tensor(dy, "dy", "f32", z.f32), _tensor(w_gate, "w_gate", "bf16", z.w_ffn),
            _tensor(w_up, "w_up", "bf16", z.w_ffn), _tensor(w_down, "w_down", "bf16", z.w_ffn)]
    if kept:
        args.append(_tensor(gu_keep, "gu_keep", "f32", tsp_workspace_bytes(dims, TSP_FN_GU)))
    args += [_tensor(dx_residual, "dx_residual", "f32", z.f32, optional=True), _tensor(dx, "dx", "f32", z.f32),
             _tensor(dw_gate, "dw_gate", "f32", fw), _tensor(dw_up, "dw_up", "f32", fw),
             _tensor(dw_down, "dw_down", "f32", fw), wsp, wsn, _s(stream)]
    _check(getattr(load(), fn)(*args))


def tsp_mlp_ring_bwd(dims, x, dy, w_gate, w_up, w_down, dx, dw_gate, dw_up, dw_down, ws, dx_residual=None,
                     x_dtype=None, stream=None):
    """Backward of the MLP ring: dx = dx_residual + dMLP/dx^T dy and this rank's
    contributions to dW_gate, dW_up ([F][h]) and dW_down ([D][h][F/D])."""
    _mlp_bwd("tsp_mlp_ring_bwd", dims, x, dy, w_gate, w_up, w_down, dx, dw_gate, dw_up, dw_down, ws, dx_residual,
             x_dtype, stream)


def tsp_mlp_ring_bwd_kept(dims, x, dy, w_gate, w_up, w_down, gu_keep, dx, dw_gate, dw_up, dw_down, ws,
                          dx_residual=None, x_dtype=None, stream=None):
    """tsp_mlp_ring_bwd from the g and u tsp_mlp_ring_fwd_keep kept (no
    recomputation of the gate/up product); the same outputs."""
    _mlp_bwd("tsp_mlp_ring_bwd_kept", dims, x, dy, w_gate, w_up, w_down, dx, dw_gate, dw_up, dw_down, ws,
             dx_residual, x_dtype, stream, gu_keep)


def tsp_attn_bwd(dims, x_local, w_qkv, w_o, kv_gathered, dh, dq, dkv_send, dw_o, ws, stream=None):
    """Attention backward before the K/V-gradient reduce-scatter: dq, the rank's
    contribution to every key's dK/dV (grouped by owner rank) and its dW_O share."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_ATTN_BWD)
    _check(load().tsp_attn_bwd(
        ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16), _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv),
        _tensor(w_o, "w_o", "bf16", z.w_o),
        _tensor(kv_gathered, "kv_gathered", "f16", tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
        _tensor(dh, "dh", "f32", z.f32), _tensor(dq, "dq", "f32", z.dq),
        _tensor(dkv_send, "dkv_send", "f32", tsp_workspace_bytes(dims, TSP_FN_DKV)),
        _tensor(dw_o, "dw_o", "f32", 2 * z.w_o), wsp, wsn, _s(stream)))


def tsp_attn_fwd_keep(dims, x_local, w_qkv, w_o, kv_gathered, out, q_keep, o_keep, lse_keep, ws, residual=None,
                      stream=None):
    """tsp_attn_fwd that also hands Q (f16 [B][Hq][T][dh]), the attention output
    O (f16 [B][T][Hq*dh]) and each row's log2 softmax normaliser (float32
    [B][Hq][T]) to the caller, for tsp_attn_bwd_kept."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_ATTN_KEEP)
    _check(load().tsp_attn_fwd_keep(
        ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16), _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv),
        _tensor(w_o, "w_o", "bf16", z.w_o),
        _tensor(kv_gathered, "kv_gathered", "f16", tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
        _tensor(residual, "residual", "f32", z.f32, optional=True), _tensor(out, "out", "f32", z.f32),
        _tensor(q_keep, "q_keep", "f16", z.q), _tensor(o_keep, "o_keep", "f16", z.q),
        _tensor(lse_keep, "lse_keep", "f32", tsp_workspace_bytes(dims, TSP_FN_LSE)), wsp, wsn, _s(stream)))


def tsp_attn_bwd_kept(dims, w_o, kv_gathered, q_keep, o_keep, lse_keep, dh, dq, dkv_send, dw_o, ws, stream=None):
    """tsp_attn_bwd from the activations tsp_attn_fwd_keep kept (no
    recomputation of Q and of the attention); the same outputs."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_ATTN_BWD_KEPT)
    _check(load().tsp_attn_bwd_kept(
        ctypes.byref(d), _tensor(w_o, "w_o", "bf16", z.w_o),
        _tensor(kv_gathered, "kv_gathered", "f16", tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
        _tensor(q_keep, "q_keep", "f16", z.q), _tensor(o_keep, "o_keep", "f16", z.q),
        _tensor(lse_keep, "lse_keep", "f32", tsp_workspace_bytes(dims, TSP_FN_LSE)),
        _tensor(dh, "dh", "f32", z.f32), _tensor(dq, "dq", "f32", z.dq),
        _tensor(dkv_send, "dkv_send", "f32", tsp_workspace_bytes(dims, TSP_FN_DKV)),
        _tensor(dw_o, "dw_o", "f32", 2 * z.w_o), wsp, wsn, _s(stream)))


def tsp_attn_bwd_proj(dims, x_local, w_qkv, dq, dkv_own, dx, dw_qkv, ws, dx_residual=None, stream=None):
    """Attention backward after the reduce-scatter: dx = dx_residual + dQ W_Q + dK W_K
    + dV W_V and the rank's share of the packed dW_QKV."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_ATTN_BWD_PROJ)
    _check(load().tsp_attn_bwd_proj(
        ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16), _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv),
        _tensor(dq, "dq", "f32", z.dq), _tensor(dkv_own, "dkv_own", "f32", z.dkv_own),
        _tensor(dx_residual, "dx_residual", "f32", z.f32, optional=True), _tensor(dx, "dx", "f32", z.f32),
        _tensor(dw_qkv, "dw_qkv", "f32", 2 * z.w_qkv), wsp, wsn, _s(stream)))


def tsp_layer_fwd(dims, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, ws, stream=None):
    z = _Sizes(dims)
    d = dims_struct(dims)
    wsp, wsn = _ws(dims, ws, TSP_FN_LAYER)
    _check(load().tsp_layer_fwd(ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16),
                                _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv), _tensor(w_o, "w_o", "bf16", z.w_o),
                                _tensor(w_gate, "w_gate", "bf16", z.w_ffn), _tensor(w_up, "w_up", "bf16", z.w_ffn),
                                _tensor(w_down, "w_down", "bf16", z.w_ffn),
                                _tensor(kv_gathered, "kv_gathered", "f16",
                                        tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
                                _tensor(y, "y", "f32", z.f32), wsp, wsn, _s(stream)))


def tsp_layer_fwd_noalloc(dims, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, stream=None):
    """tsp_layer_fwd on the library's fixed scratch array (no workspace, no allocation)."""
    z = _Sizes(dims)
    d = dims_struct(dims)
    _check(load().tsp_layer_fwd_noalloc(
        ctypes.byref(d), _tensor(x_local, "x_local", "bf16", z.x16), _tensor(w_qkv, "w_qkv", "bf16", z.w_qkv),
        _tensor(w_o, "w_o", "bf16", z.w_o), _tensor(w_gate, "w_gate", "bf16", z.w_ffn),
        _tensor(w_up, "w_up", "bf16", z.w_ffn), _tensor(w_down, "w_down", "bf16", z.w_ffn),
        _tensor(kv_gathered, "kv_gathered", "f16", tsp_workspace_bytes(dims, TSP_FN_KV_GATHERED)),
        _tensor(y, "y", "f32", z.f32), _s(stream)))


def tsp_set_tuning(knob, value: int | None):
    """Kernel-choice override for tests and tuning: knob name (see TUNE) or id;
    value None or < 0 restores the default dispatch."""
    kid = TUNE[knob] if isinstance(knob, str) else int(knob)
    _check(load().tsp_set_tuning(kid, -1 if value is None else int(value)))


def reset_tuning():
    for kid in TUNE.values():
        load().tsp_set_tuning(kid, -1)


def tsp_profile_kernel(kernel, max_launches: int = 1):
    """Arm live HIP-event timing of the next launches of one kernel ('qkv', 'reorder',
    'attn', 'oproj', 'gateup', 'down', 'attn_bwd'; None disarms)."""
    kid = 0 if kernel is None else KERNELS[kernel]
    _check(load().tsp_profile_kernel(kid, int(max_launches)))


def tsp_profile_result():
    """(launches, total_ms) of the armed kernel since the last read."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_float(0.0)
    _check(load().tsp_profile_result(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
