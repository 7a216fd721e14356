"""ctypes binding of libtsp.so: same names as the C ABI, argument marshalling only.

Every computation happens in the HIP kernels behind the C ABI; this module
turns torch tensors into device pointers and the current HIP stream into a
``hipStream_t``.  If the library is not built it raises -- there is no CPU
fallback.
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

TSP_FN_ATTN = 1
TSP_FN_MLP = 2
TSP_FN_LAYER = 3
TSP_FN_KV_NATURAL = 4
TSP_FN_KV_GATHERED = 5

KERNELS = {"qkv": 1, "reorder": 2, "attn": 3, "oproj": 4, "gateup": 5, "down": 6}

EXPORTED = ("tsp_zigzag_index", "tsp_qkv_proj", "tsp_kv_reorder", "tsp_attn_fwd",
            "tsp_mlp_ring_fwd", "tsp_layer_fwd", "tsp_workspace_bytes", "tsp_last_error",
            "tsp_profile_kernel", "tsp_profile_result")


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
        "tsp_kv_reorder": [dp, vp, vp, vp],
        "tsp_attn_fwd": [dp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_mlp_ring_fwd": [dp, vp, vp, vp, vp, vp, vp, sz, vp],
        "tsp_layer_fwd": [dp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
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


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


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


def tsp_zigzag_index(dims, local_to_global, global_to_slot=None, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_zigzag_index(ctypes.byref(d), _p(local_to_global), _p(global_to_slot), _s(stream)))


def tsp_qkv_proj(dims, src_rank, x_shard, w_qkv, q_out, kv_gathered, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_qkv_proj(ctypes.byref(d), int(src_rank), _p(x_shard), _p(w_qkv), _p(q_out),
                               _p(kv_gathered), _s(stream)))


def tsp_kv_reorder(dims, kv_gathered, kv_natural, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_kv_reorder(ctypes.byref(d), _p(kv_gathered), _p(kv_natural), _s(stream)))


def tsp_attn_fwd(dims, x_local, w_qkv, w_o, kv_gathered, out, ws, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_attn_fwd(ctypes.byref(d), _p(x_local), _p(w_qkv), _p(w_o), _p(kv_gathered),
                               _p(out), _p(ws), _nbytes(ws), _s(stream)))


def tsp_mlp_ring_fwd(dims, x, w_gate, w_up, w_down, y, ws, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_mlp_ring_fwd(ctypes.byref(d), _p(x), _p(w_gate), _p(w_up), _p(w_down), _p(y),
                                   _p(ws), _nbytes(ws), _s(stream)))


def tsp_layer_fwd(dims, x_local, w_qkv, w_o, w_gate, w_up, w_down, kv_gathered, y, ws, stream=None):
    d = dims_struct(dims)
    _check(load().tsp_layer_fwd(ctypes.byref(d), _p(x_local), _p(w_qkv), _p(w_o), _p(w_gate), _p(w_up),
                                _p(w_down), _p(kv_gathered), _p(y), _p(ws), _nbytes(ws), _s(stream)))


def tsp_profile_kernel(kernel, max_launches: int = 1):
    """Arm live HIP-event timing of the next launches of one kernel ('qkv', 'reorder',
    'attn', 'oproj', 'gateup', 'down'; None disarms)."""
    kid = 0 if kernel is None else KERNELS[kernel]
    _check(load().tsp_profile_kernel(kid, int(max_launches)))


def tsp_profile_result():
    """(launches, total_ms) of the armed kernel since the last read."""
    n = ctypes.c_int32(0)
    ms = ctypes.c_float(0.0)
    _check(load().tsp_profile_result(ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value
