"""Device-side set-up of one rank's TSP layer problem (marshalling only).

Packs the unsharded nn.Linear-style weights into the per-shard layouts of the
C ABI, uploads them, builds the rank's local rows with the library's own
zigzag index kernel, and fills the other ranks' slots of the K/V all-gather
buffer by calling ``tsp_qkv_proj`` once per other rank (this stands in for the
all-gather having arrived; it is not part of the timed layer).
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

from . import binding as B


def _u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


def pack_weights(inputs: dict, dims) -> dict:
    """bf16 bit arrays in ABI layouts (host torch int16 tensors).

    w_qkv [D][(Hq/D + 2 Hkv/D) dh][h]: shard j = its q-heads, k-heads, v-heads;
    w_o [D][h][Hq/D dh]; w_gate, w_up [F][h]; w_down [D][h][F/D].
    """
    D, dh = dims.degree, dims.head_dim
    hq_s, hkv_s, f_s = dims.n_q_heads // D, dims.n_kv_heads // D, dims.ffn // D
    wq, wk, wv, wo, wd = (inputs[n] for n in ("w_q", "w_k", "w_v", "w_o", "w_d"))
    qkv = np.stack([np.concatenate([wq[j * hq_s * dh:(j + 1) * hq_s * dh],
                                    wk[j * hkv_s * dh:(j + 1) * hkv_s * dh],
                                    wv[j * hkv_s * dh:(j + 1) * hkv_s * dh]]) for j in range(D)])
    o = np.stack([wo[:, j * hq_s * dh:(j + 1) * hq_s * dh] for j in range(D)])
    down = np.stack([wd[:, j * f_s:(j + 1) * f_s] for j in range(D)])
    return {"w_qkv": _u16(qkv), "w_o": _u16(o), "w_gate": _u16(inputs["w_g"]),
            "w_up": _u16(inputs["w_u"]), "w_down": _u16(down)}


@dataclasses.dataclass
class RankProblem:
    dims: object
    w: dict                 # device weights (ABI layouts)
    x_full: torch.Tensor    # bf16 bits [B][S][h] on device
    l2g: dict               # rank -> int32 device tensor [T]
    x_local: torch.Tensor   # bf16 bits [B][T][h] of dims.rank
    kv_gathered: torch.Tensor
    ws: torch.Tensor
    y: torch.Tensor

    @classmethod
    def build(cls, dims, inputs: dict, device="cuda", stream=None, fill_other_ranks=True):
        w = {k: v.to(device) for k, v in pack_weights(inputs, dims).items()}
        x_full = _u16(inputs["x"]).to(device)
        l2g = {}
        D = dims.degree
        T = dims.seq // D
        for r in range(D):
            dr = dataclasses.replace(dims, rank=r)
            t = torch.empty(T, dtype=torch.int32, device=device)
            B.tsp_zigzag_index(dr, t, None, stream)
            l2g[r] = t
        x_loc = {r: x_full.index_select(1, l2g[r].long()).contiguous() for r in range(D)}
        nkv = B.tsp_workspace_bytes(dims, B.TSP_FN_KV_GATHERED) // 2
        kv = torch.zeros(nkv, dtype=torch.int16, device=device)
        if fill_other_ranks:
            for r in range(D):
                if r != dims.rank:
                    B.tsp_qkv_proj(dataclasses.replace(dims, rank=r), r, x_loc[r], w["w_qkv"], None,
                                   kv, stream)
        ws = torch.empty(B.tsp_workspace_bytes(dims, B.TSP_FN_LAYER), dtype=torch.uint8, device=device)
        y = torch.empty((dims.batch, T, dims.hidden), dtype=torch.float32, device=device)
        return cls(dims, w, x_full, l2g, x_loc[dims.rank], kv, ws, y)

    def layer(self, stream=None):
        w = self.w
        B.tsp_layer_fwd(self.dims, self.x_local, w["w_qkv"], w["w_o"], w["w_gate"], w["w_up"],
                        w["w_down"], self.kv_gathered, self.y, self.ws, stream)
        return self.y
