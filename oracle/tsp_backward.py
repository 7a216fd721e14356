"""Plain CPU float64 oracle for the backward pass of the TSP transformer layer.

TEST INFRASTRUCTURE ONLY, under the rules of ``tsp_oracle``: only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the HIP library never routes through it and shares no code with it.

What is computed, and where the pages define it
-----------------------------------------------
TSP is presented as a scheme for training as well as serving (Zyphra TSP
article on ai-trends.today, opening paragraph and section "What you need to
know"; aivizor.me news post, second paragraph), but the pages describe only
the forward schedules.  The backward computed here is the plain gradient of
the forward layer of ``tsp_oracle`` (h = x + Attn(x), y = h + MLP(h)) with
respect to its input and its seven weight matrices, for a given upstream
gradient dY:

    layer_backward        the unsharded layer's gradients, float64 (the
                          reference result);
    mlp_backward          the gated MLP's gradients on given rows;
    attention_backward    causal softmax attention's gradients for one head;
    tsp_backward_schedule the backward run as a TSP schedule over D virtual
                          ranks (the transpose of the forward schedule, read
                          below), used to show that the schedule reproduces
                          the unsharded gradients.

The TSP backward schedule (the reading taken; the pages give none).  Every
exchange of the forward schedule is reversed:
  * MLP ring: the shards travel round the ring again, each together with an
    accumulator of its weight gradients; at each step a rank adds the
    contribution of its own tokens to the shard it holds, so after D steps
    every accumulator is back at its owner holding the sum over all ranks.
    The input gradient stays local: dH += dG_j W_g,j + dU_j W_u,j summed over
    the shards, as the forward summed the shards' outputs (the transpose of a
    row split is a column split: bowenzhou.top "张量并行", section
    "机制：行切与列切").
  * Attention: for each shard j, the rank recomputes its queries' attention
    over all keys; the gradients it produces for every key's K and V rows
    are reduce-scattered back to the ranks that own those tokens (the
    transpose of the all-gather); each rank then forms its share of the
    weight gradients of W_Q, W_K, W_V and W_O from its own tokens, and these
    shares are summed at the shard's owner (the transpose of the broadcast).

Gradient formulas (standard calculus; nothing is approximated):
  silu'(z) = s (1 + z (1 - s)),  s = 1 / (1 + e^-z);
  softmax rows: dS = P * (dP - rowsum(dP * P)), dP = dO V^T.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from .tsp_oracle import _dims, _part, bf16_bits_to_f64, causal_attention, global_to_slot, local_to_global, silu

__all__ = ["sigmoid", "silu_grad", "mlp_backward", "attention_backward", "layer_backward",
           "rank_mlp_backward", "tsp_backward_schedule", "rank_attention_bwd_queries", "rank_attention_bwd_proj",
           "reduce_scatter_dkv", "rank_attention_backward"]

WEIGHTS = ("w_q", "w_k", "w_v", "w_o", "w_g", "w_u", "w_d")


def sigmoid(z: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-z) without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d/dz [z s(z)] = s (1 + z (1 - s))."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def mlp_backward(x: np.ndarray, w_g: np.ndarray, w_u: np.ndarray, w_d: np.ndarray, dy: np.ndarray) -> dict:
    """Gradients of m = (silu(x Wg^T) * (x Wu^T)) Wd^T for rows x [n][h] given
    dm = dy [n][h]: dx (the MLP branch only, no residual), dw_g, dw_u [F][h],
    dw_d [h][F], plus the forward intermediates g, u, a."""
    g = x @ w_g.T
    u = x @ w_u.T
    sg = silu(g)
    a = sg * u
    da = dy @ w_d                       # [n][F]
    du = da * sg
    dg = da * u * silu_grad(g)
    return {"dx": dg @ w_g + du @ w_u, "dw_g": dg.T @ x, "dw_u": du.T @ x, "dw_d": dy.T @ a,
            "g": g, "u": u, "a": a, "dg": dg, "du": du, "da": da}


def attention_backward(q, k, v, q_pos, do, scale=None, block=256):
    """Gradients of o[i] = sum_{j <= q_pos[i]} softmax_j(q[i].k[j] scale) v[j]
    for one head: returns dq [n][dh], dk and dv shaped like k and v (only the
    keys the queries reach get non-zero rows)."""
    q = np.asarray(q, dtype=np.float64)
    dh = q.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    q_pos = np.asarray(q_pos, dtype=np.int64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    for i0 in range(0, q.shape[0], block):
        i1 = min(q.shape[0], i0 + block)
        pos = q_pos[i0:i1]
        nk = int(pos.max()) + 1
        s = (q[i0:i1] @ k[:nk].T) * scale
        s[np.arange(nk)[None, :] > pos[:, None]] = -np.inf
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        dov = do[i0:i1]
        dv[:nk] += p.T @ dov
        dp = dov @ v[:nk].T
        ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))
        dq[i0:i1] = (ds @ k[:nk]) * scale
        dk[:nk] += (ds.T @ q[i0:i1]) * scale
    return dq, dk, dv


def _weights(inputs):
    return {n: bf16_bits_to_f64(inputs[n]) for n in WEIGHTS}


def layer_backward(inputs: dict, dims, dy: np.ndarray, weights=None) -> dict:
    """Gradients of the unsharded layer over whole sequences.

    dy: float [B][S][h], the gradient of y.  Returns dx [B][S][h], dh (the
    gradient at h = x + Attn(x)) and the seven weight gradients (same shapes
    as the weights), all float64.
    """
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    w = _weights(inputs) if weights is None else weights
    grads = {n: np.zeros_like(w[n]) for n in WEIGHTS}
    dx_all = np.empty((B, S, h))
    dh_all = np.empty((B, S, h))
    group = Hq // Hkv
    pos = np.arange(S)
    for b in range(B):
        x = bf16_bits_to_f64(inputs["x"][b])
        q, k, v = x @ w["w_q"].T, x @ w["w_k"].T, x @ w["w_v"].T
        o = np.empty((S, Hq * dh))
        for i in range(Hq):
            kvh = i // group
            o[:, i * dh:(i + 1) * dh] = causal_attention(q[:, i * dh:(i + 1) * dh], k[:, kvh * dh:(kvh + 1) * dh],
                                                         v[:, kvh * dh:(kvh + 1) * dh], pos)
        hres = x + o @ w["w_o"].T
        dyb = np.asarray(dy[b], dtype=np.float64)
        m = mlp_backward(hres, w["w_g"], w["w_u"], w["w_d"], dyb)
        grads["w_g"] += m["dw_g"]
        grads["w_u"] += m["dw_u"]
        grads["w_d"] += m["dw_d"]
        dhres = dyb + m["dx"]
        dh_all[b] = dhres
        grads["w_o"] += dhres.T @ o
        do = dhres @ w["w_o"]
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for i in range(Hq):
            kvh = i // group
            sl, kl = slice(i * dh, (i + 1) * dh), slice(kvh * dh, (kvh + 1) * dh)
            gq, gk, gv = attention_backward(q[:, sl], k[:, kl], v[:, kl], pos, do[:, sl])
            dq[:, sl] = gq
            dk[:, kl] += gk
            dv[:, kl] += gv
        grads["w_q"] += dq.T @ x
        grads["w_k"] += dk.T @ x
        grads["w_v"] += dv.T @ x
        dx_all[b] = dhres + dq @ w["w_q"] + dk @ w["w_k"] + dv @ w["w_v"]
    out = {"dx": dx_all, "dh": dh_all}
    out.update({"d" + n: g for n, g in grads.items()})
    return out


def rank_mlp_backward(x_rows: np.ndarray, dy_rows: np.ndarray, inputs: dict, dims) -> dict:
    """One rank's share of the MLP ring backward: its tokens' input gradient
    (the MLP branch, summed over the D shards in ring order (r - s) mod D)
    and its contribution to every shard's weight gradients, in the forward
    layouts (w_g, w_u [F][h] = [D][F/D][h]; w_d [h][F] sliced per shard)."""
    D, r, F = dims.degree, dims.rank, dims.ffn
    fs = F // D
    w = {n: bf16_bits_to_f64(inputs[n]) for n in ("w_g", "w_u", "w_d")}
    dx = np.zeros_like(x_rows)
    dw_g = np.zeros_like(w["w_g"])
    dw_u = np.zeros_like(w["w_u"])
    dw_d = np.zeros_like(w["w_d"])
    for s in range(D):
        j = (r - s) % D
        cols = slice(j * fs, (j + 1) * fs)
        m = mlp_backward(x_rows, w["w_g"][cols], w["w_u"][cols], w["w_d"][:, cols], dy_rows)
        dx += m["dx"]
        dw_g[cols], dw_u[cols], dw_d[:, cols] = m["dw_g"], m["dw_u"], m["dw_d"]
    return {"dx": dx, "dw_g": dw_g, "dw_u": dw_u, "dw_d": dw_d}


def tsp_backward_schedule(inputs: dict, dims, dy: np.ndarray) -> dict:
    """The backward as a TSP schedule over all D virtual ranks (exchanges are
    array copies).  dy: [B][S][h] in sequence order.  Returns dx [B][S][h]
    reassembled in sequence order and the seven weight gradients as the
    shard owners hold them after the schedule (summed over ranks)."""
    B, S, D, _r, h, Hq, Hkv, dh, F = _dims(dims)
    T = S // D
    hq_s, hkv_s, fs = Hq // D, Hkv // D, F // D
    w = _weights(inputs)
    x_all = bf16_bits_to_f64(inputs["x"])
    l2g = [local_to_global(S, D, r, _part(dims)) for r in range(D)]
    slot = global_to_slot(S, D, _part(dims))
    x_loc = [x_all[:, l2g[r]] for r in range(D)]
    dy_loc = [np.asarray(dy, dtype=np.float64)[:, l2g[r]] for r in range(D)]
    group = Hq // Hkv

    # ---- forward again (each rank keeps its own activations) -------------
    o_loc = [np.zeros((B, T, Hq * dh)) for _ in range(D)]
    kv_nat = {}
    for j in range(D):
        qr, kr = slice(j * hq_s * dh, (j + 1) * hq_s * dh), slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        k_gath = np.concatenate([x_loc[r] @ w["w_k"][kr].T for r in range(D)], axis=1)
        v_gath = np.concatenate([x_loc[r] @ w["w_v"][kr].T for r in range(D)], axis=1)
        kv_nat[j] = (k_gath[:, slot], v_gath[:, slot])
        for r in range(D):
            qj = x_loc[r] @ w["w_q"][qr].T
            for b in range(B):
                for i in range(hq_s):
                    kvh = (j * hq_s + i) // group - j * hkv_s
                    o_loc[r][b, :, qr][:, i * dh:(i + 1) * dh] = causal_attention(
                        qj[b, :, i * dh:(i + 1) * dh], kv_nat[j][0][b, :, kvh * dh:(kvh + 1) * dh],
                        kv_nat[j][1][b, :, kvh * dh:(kvh + 1) * dh], l2g[r])
    h_loc = [x_loc[r] + o_loc[r] @ w["w_o"].T for r in range(D)]

    # ---- MLP ring backward: accumulators travel with the shards ----------
    acc = {j: {"w_g": np.zeros((fs, h)), "w_u": np.zeros((fs, h)), "w_d": np.zeros((h, fs))} for j in range(D)}
    held = list(range(D))                     # shard held by rank r at step s: (r - s) mod D
    dh_loc = [dy_loc[r].copy() for r in range(D)]
    for s in range(D):
        for r in range(D):
            j = held[r]
            cols = slice(j * fs, (j + 1) * fs)
            for b in range(B):
                m = mlp_backward(h_loc[r][b], w["w_g"][cols], w["w_u"][cols], w["w_d"][:, cols], dy_loc[r][b])
                dh_loc[r][b] += m["dx"]
                acc[j]["w_g"] += m["dw_g"]
                acc[j]["w_u"] += m["dw_u"]
                acc[j]["w_d"] += m["dw_d"]
        held = [held[(r - 1) % D] for r in range(D)]   # pass shard and accumulator to rank r + 1

    # ---- attention backward per shard -------------------------------------
    dx_loc = [dh_loc[r].copy() for r in range(D)]
    grads = {n: np.zeros_like(w[n]) for n in ("w_q", "w_k", "w_v", "w_o")}
    for j in range(D):
        qr, kr = slice(j * hq_s * dh, (j + 1) * hq_s * dh), slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        k_nat, v_nat = kv_nat[j]
        dk_from = np.zeros((D, B, S, hkv_s * dh))          # rank r's queries -> every key
        dv_from = np.zeros((D, B, S, hkv_s * dh))
        dq_loc = [np.zeros((B, T, hq_s * dh)) for _ in range(D)]
        for r in range(D):
            grads["w_o"][:, qr] += np.einsum("bth,btk->hk", dh_loc[r], o_loc[r][:, :, qr])   # W_O share
            do = dh_loc[r] @ w["w_o"][:, qr]
            qj = x_loc[r] @ w["w_q"][qr].T
            for b in range(B):
                for i in range(hq_s):
                    kvh = (j * hq_s + i) // group - j * hkv_s
                    sl, kl = slice(i * dh, (i + 1) * dh), slice(kvh * dh, (kvh + 1) * dh)
                    gq, gk, gv = attention_backward(qj[b, :, sl], k_nat[b, :, kl], v_nat[b, :, kl], l2g[r],
                                                    do[b, :, sl])
                    dq_loc[r][b, :, sl] = gq
                    dk_from[r, b, :, kl] += gk
                    dv_from[r, b, :, kl] += gv
        # reduce-scatter of the K/V gradients back to the tokens' owners
        dk_tot, dv_tot = dk_from.sum(axis=0), dv_from.sum(axis=0)
        for r in range(D):
            dk_r, dv_r = dk_tot[:, l2g[r]], dv_tot[:, l2g[r]]
            grads["w_q"][qr] += np.einsum("btk,bth->kh", dq_loc[r], x_loc[r])
            grads["w_k"][kr] += np.einsum("btk,bth->kh", dk_r, x_loc[r])
            grads["w_v"][kr] += np.einsum("btk,bth->kh", dv_r, x_loc[r])
            dx_loc[r] += dq_loc[r] @ w["w_q"][qr] + dk_r @ w["w_k"][kr] + dv_r @ w["w_v"][kr]

    dx = np.empty((B, S, h))
    for r in range(D):
        dx[:, l2g[r]] = dx_loc[r]
    out = {"dx": dx, "dw_q": grads["w_q"], "dw_k": grads["w_k"], "dw_v": grads["w_v"], "dw_o": grads["w_o"]}
    out["dw_g"] = np.concatenate([acc[j]["w_g"] for j in range(D)])
    out["dw_u"] = np.concatenate([acc[j]["w_u"] for j in range(D)])
    out["dw_d"] = np.concatenate([acc[j]["w_d"] for j in range(D)], axis=1)
    return out


# --------------------------------------------------------------------------- #
# One rank's share of the attention backward (the pieces of the schedule above
# that rank r computes, for the per-kernel tests)
# --------------------------------------------------------------------------- #
def rank_attention_bwd_queries(inputs: dict, dims, dh_rows: np.ndarray) -> dict:
    """The part of rank dims.rank's attention backward that comes before the
    reduce-scatter, from the gradient at h = x + Attn(x) of its own tokens
    (dh_rows [B][T][h], local row order):

      dq          [B][T][Hq*dh]   its queries' gradient (unscaled Q space)
      dkv_contrib [D][2][B][S][Hkv/D*dh]  its queries' contribution to every
                  key's K and V gradient, per shard j, keys in sequence order
                  (what the reduce-scatter sums over ranks)
      dw_o        [h][Hq*dh]      its tokens' share of dW_O
      do, o       [B][T][Hq*dh]   the output gradient dh W_O and the
                  recomputed attention output
    """
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    T = S // D
    hkv_s = Hkv // D
    w = _weights(inputs)
    x_all = bf16_bits_to_f64(inputs["x"])
    rows = local_to_global(S, D, r, _part(dims))
    group = Hq // Hkv
    k_all = x_all @ w["w_k"].T          # [B][S][Hkv*dh]
    v_all = x_all @ w["w_v"].T
    q = x_all[:, rows] @ w["w_q"].T
    dhr = np.asarray(dh_rows, dtype=np.float64)
    do = dhr @ w["w_o"]
    dq = np.zeros((B, T, Hq * dh))
    dk = np.zeros((B, S, Hkv * dh))
    dv = np.zeros((B, S, Hkv * dh))
    o = np.zeros((B, T, Hq * dh))
    for b in range(B):
        for i in range(Hq):
            kvh = i // group
            sl, kl = slice(i * dh, (i + 1) * dh), slice(kvh * dh, (kvh + 1) * dh)
            o[b, :, sl] = causal_attention(q[b, :, sl], k_all[b, :, kl], v_all[b, :, kl], rows)
            gq, gk, gv = attention_backward(q[b, :, sl], k_all[b, :, kl], v_all[b, :, kl], rows, do[b, :, sl])
            dq[b, :, sl] = gq
            dk[b, :, kl] += gk
            dv[b, :, kl] += gv
    dkv_contrib = np.zeros((D, 2, B, S, hkv_s * dh))
    for j in range(D):
        kl = slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        dkv_contrib[j, 0], dkv_contrib[j, 1] = dk[:, :, kl], dv[:, :, kl]
    dw_o = dhr.reshape(-1, h).T @ o.reshape(-1, Hq * dh)
    return {"dq": dq, "dkv_contrib": dkv_contrib, "dw_o": dw_o, "do": do, "o": o}


def rank_attention_bwd_proj(inputs: dict, dims, dq: np.ndarray, dkv_own: np.ndarray) -> dict:
    """The part after the reduce-scatter, from the rank's query gradient dq
    [B][T][Hq*dh] and the K/V gradient of its own tokens summed over every
    rank's queries (dkv_own [D][2][B][T][Hkv/D*dh], per shard j):

      dw_qkv  [D][(Hq/D + 2 Hkv/D)*dh][h]  its tokens' share of the packed
              Q/K/V weight gradients (the tsp_qkv_proj packing)
      dx_attn [B][T][h]  the attention branch's input gradient
              dQ W_Q + dK W_K + dV W_V (the residual's dh not added)
    """
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    hq_s, hkv_s = Hq // D, Hkv // D
    w = _weights(inputs)
    x = bf16_bits_to_f64(inputs["x"])[:, local_to_global(S, D, r, _part(dims))]
    dq = np.asarray(dq, dtype=np.float64)
    dkv_own = np.asarray(dkv_own, dtype=np.float64)
    dk_own = np.concatenate([dkv_own[j, 0] for j in range(D)], axis=2)   # [B][T][Hkv*dh]
    dv_own = np.concatenate([dkv_own[j, 1] for j in range(D)], axis=2)
    dw_qkv = np.zeros((D, (hq_s + 2 * hkv_s) * dh, h))
    for j in range(D):
        ql, kl = slice(j * hq_s * dh, (j + 1) * hq_s * dh), slice(j * hkv_s * dh, (j + 1) * hkv_s * dh)
        g = np.concatenate([dq[:, :, ql], dk_own[:, :, kl], dv_own[:, :, kl]], axis=2)   # [B][T][nqkv_s]
        dw_qkv[j] = g.reshape(-1, g.shape[2]).T @ x.reshape(-1, h)
    dx_attn = dq @ w["w_q"] + dk_own @ w["w_k"] + dv_own @ w["w_v"]
    return {"dw_qkv": dw_qkv, "dx_attn": dx_attn}


def reduce_scatter_dkv(contribs: list, dims) -> np.ndarray:
    """The reduce-scatter of the K/V gradients: rank dims.rank's own tokens'
    rows of the D ranks' contributions ([D][2][B][S][Hkv/D*dh] each), summed
    -> [D][2][B][T][Hkv/D*dh]."""
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    rows = local_to_global(S, D, r, _part(dims))
    return sum(np.asarray(c, dtype=np.float64)[:, :, :, rows] for c in contribs)


def rank_attention_backward(inputs: dict, dims, dh_all: np.ndarray) -> dict:
    """Rank dims.rank's whole share of the attention backward, given the
    gradient at h = x + Attn(x) for every token (dh_all [B][S][h], sequence
    order): the entries of rank_attention_bwd_queries for its own tokens,
    dkv_own (the reduce-scatter of every rank's contribution) and the entries
    of rank_attention_bwd_proj."""
    B, S, D, r, h, Hq, Hkv, dh, F = _dims(dims)
    part = _part(dims)
    dh_all = np.asarray(dh_all, dtype=np.float64)
    shares = []
    for rq in range(D):
        drq = _with_rank(dims, rq)
        shares.append(rank_attention_bwd_queries(inputs, drq, dh_all[:, local_to_global(S, D, rq, part)]))
    own = shares[r]
    dkv_own = reduce_scatter_dkv([sh["dkv_contrib"] for sh in shares], dims)
    out = dict(own)
    out["dkv_own"] = dkv_own
    out.update(rank_attention_bwd_proj(inputs, dims, own["dq"], dkv_own))
    return out


def _with_rank(dims, rank):
    return dataclasses.replace(dims, rank=rank)
