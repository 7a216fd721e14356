"""MI355X-native per-rank Tensor-and-Sequence-Parallel (TSP) layer forward.

The compute lives in libtsp.so (HIP kernels for gfx950 behind a C ABI, see
include/tsp.h); ``binding`` exposes the same entry points to Python and
``harness`` sets up a rank's device problem.
"""
from .binding import (  # noqa: F401
    TSP_BF16, TSP_F16, TSP_F32, TSP_FN_ATTN, TSP_FN_KV_GATHERED, TSP_FN_KV_NATURAL, TSP_FN_LAYER,
    TSP_FN_MLP, TspDims, TspError, load, tsp_attn_bwd, tsp_attn_bwd_kept, tsp_attn_bwd_proj, tsp_attn_fwd,
    tsp_attn_fwd_keep, tsp_kv_reorder, tsp_layer_fwd, tsp_mlp_ring_bwd, tsp_mlp_ring_bwd_kept, tsp_mlp_ring_fwd,
    tsp_mlp_ring_fwd_keep, tsp_qkv_proj, tsp_set_tuning, tsp_workspace_bytes, tsp_zigzag_index)
