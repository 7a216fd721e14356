"""Analytic per-GPU peak training memory of TSP, TP and TP x SP layouts.

A calculator, host-only: it runs nothing on the GPU.  Parity with the pages
is partly pinned: the pages give totals, not a breakdown (see below).

What the pages fix
------------------
* Model state.  Mixed-precision Adam keeps 16 bytes per parameter: 16-bit
  weights (2) and gradients (2), float32 master weights, momentum and
  variance (12); a 7B model therefore needs 112 GB of training state
  (r007.github.io "Распределенное обучение", section "Эффективный по памяти
  параллелизм по данным: ZeRO и FSDP", worked example "ZeRO: экономия
  памяти").
* TSP.  Every rank of a TSP axis of size D holds 1/D of every weight matrix
  and 1/D of the sequence, so both the weight-proportional memory
  (parameters, gradients, optimizer state) and the activation memory drop by
  1/D (ai-trends.today TSP article, section "How to Fold a Book").
* TP and SP.  Tensor parallelism of degree T splits the weights (model
  state / T) but not the token dimension; sequence parallelism of degree
  Sigma splits the tokens and replicates the weights; the usual 2-D layout
  puts them on orthogonal mesh axes and needs T * Sigma devices (same
  article, section "It is TSP that solves the problem").
* Figures: the 7B dense decoder (H = 4096, 32 layers, 32 query / 32 KV
  heads, FFN factor 4, bf16) on one 8-GPU node at 128K context needs, per
  GPU, 38.8 GB with TSP, 70.0 GB with TP and 85.0-140.0 GB with TP+SP
  layouts; at short context TSP and TP are about equal because model state
  dominates (sections "Memory and Processing Results" and "What you need to
  know").

The activation model (the reading taken where the pages are silent)
--------------------------------------------------------------------
Per token and layer a layer keeps ``a_rep`` bytes that TP leaves replicated
on its T ranks (activations at the layer boundaries, where every TP rank
holds the full hidden vector of every token) and ``a_sh`` bytes that TP
splits over its ranks (per-head Q/K/V/O, per-column MLP intermediates).
Per GPU, with S tokens of context, batch B and L layers:

    TSP, degree D            16 P / D + S B L (a_rep + a_sh) / D
    TP, degree T             16 P / T + S B L (a_rep + a_sh / T)
    TP x SP, T * Sigma GPUs  16 P / T + S B L (a_rep / Sigma + a_sh / (T Sigma))

The pages give no split of their totals, so the two coefficients are
*fitted* to two of their figures (TSP 38.8 GB, TP 70.0 GB at 128K on 8
GPUs); the calculator is then checked against what was not fitted: the
TP+SP range 85.0-140.0 GB and TSP ~ TP at short context.  A first-principles
count of the tensors the layer of this library saves for its backward pass
(bf16, no recomputation) is given beside the fit for comparison, and
kept_activation_bytes gives what the library's kept-activation calls hold
per rank and layer on top of the layer inputs.
"""
from __future__ import annotations

import dataclasses

__all__ = ["Model", "Layout", "MODEL_7B", "PAGES_128K", "model_state_bytes", "per_gpu_bytes",
           "kept_activation_bytes", "fit_activation_coeffs", "first_principles_coeffs", "report"]

GB = 1e9                      # the pages' figures are decimal gigabytes (7e9 x 16 B = 112 GB)
ADAM_MIXED_BYTES_PER_PARAM = 16


@dataclasses.dataclass(frozen=True)
class Model:
    """A dense decoder: parameter count and the shapes activations depend on."""
    params: float
    hidden: int
    layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    gated: bool = True


# The pages' reference model: "7B dense", H = 4096, 32 layers, 32 q / 32 KV
# heads, FFN expansion factor 4 (read as ffn = 4 H), bf16.
MODEL_7B = Model(params=7e9, hidden=4096, layers=32, n_q_heads=32, n_kv_heads=32, head_dim=128,
                 ffn=4 * 4096, gated=True)

# The pages' per-GPU figures at 128K context on one 8-GPU node (GB).
PAGES_128K = {"seq": 131072, "devices": 8, "tsp": 38.8, "tp": 70.0, "tpsp": (85.0, 140.0)}


@dataclasses.dataclass(frozen=True)
class Layout:
    """kind: 'tsp' (degree = D), 'tp' (degree = T), 'tpsp' (degree = T, sp = Sigma)."""
    kind: str
    degree: int
    sp: int = 1

    @property
    def devices(self) -> int:
        return self.degree * self.sp


def model_state_bytes(params: float, bytes_per_param: int = ADAM_MIXED_BYTES_PER_PARAM) -> float:
    """Weights, gradients and optimizer state of `params` parameters."""
    return params * bytes_per_param


def per_gpu_bytes(layout: Layout, model: Model, seq: int, batch: int, a_rep: float, a_sh: float) -> dict:
    """Per-GPU model state, activations and their sum (bytes) for one layout."""
    tokens = float(seq) * batch * model.layers     # token-layers
    ms = model_state_bytes(model.params)
    if layout.kind == "tsp":
        d = layout.degree
        state, act = ms / d, tokens * (a_rep + a_sh) / d
    elif layout.kind == "tp":
        t = layout.degree
        state, act = ms / t, tokens * (a_rep + a_sh / t)
    elif layout.kind == "tpsp":
        t, sp = layout.degree, layout.sp
        state, act = ms / t, tokens * (a_rep / sp + a_sh / (t * sp))
    else:
        raise ValueError(f"unknown layout {layout.kind!r}")
    return {"model_state": state, "activations": act, "total": state + act}


def fit_activation_coeffs(model: Model = MODEL_7B, pages: dict = PAGES_128K, batch: int = 1):
    """(a_rep, a_sh) in bytes per token per layer that make the formulas give
    the pages' TSP and TP figures exactly (two equations, two unknowns)."""
    n = pages["devices"]
    tokens = float(pages["seq"]) * batch * model.layers
    ms = model_state_bytes(model.params) / n
    tsp_act = pages["tsp"] * GB - ms                  # = tokens (a_rep + a_sh) / n
    tp_act = pages["tp"] * GB - ms                    # = tokens (a_rep + a_sh / n)
    total = tsp_act * n / tokens                      # a_rep + a_sh
    # a_rep + (total - a_rep) / n = tp_act / tokens
    a_rep = (tp_act / tokens - total / n) / (1.0 - 1.0 / n)
    return a_rep, total - a_rep


def first_principles_coeffs(model: Model = MODEL_7B, elem_bytes: int = 2):
    """Bytes per token per layer the layer h = x + Attn(x), y = h + MLP(h) saves
    for its backward pass with nothing recomputed (flash attention keeps no
    score matrix): replicated under TP are its two inputs x and h; split under
    TP are Q, K, V, the attention output O and the MLP's gate, up and
    activation (2 of the 3 without gating)."""
    h, dh = model.hidden, model.head_dim
    rep = 2 * h * elem_bytes
    qkvo = (2 * model.n_q_heads + 2 * model.n_kv_heads) * dh * elem_bytes
    mlp = (3 if model.gated else 2) * model.ffn * elem_bytes
    return float(rep), float(qkvo + mlp)


def kept_activation_bytes(model: Model, seq: int, batch: int, degree: int) -> dict:
    """Bytes one TSP rank keeps per layer when the backward takes the
    forward's activations instead of recomputing them (the library's
    kept-activation calls): Q and the attention output O of the rank's
    S/D tokens (16-bit, all heads), each row's softmax normaliser (float32,
    per q-head), and the MLP's g and u (float32, all F columns)."""
    tokens = batch * (seq // degree)
    qo = 2 * tokens * model.n_q_heads * model.head_dim * 2
    lse = batch * model.n_q_heads * (seq // degree) * 4
    gu = 2 * tokens * model.ffn * 4
    return {"attention": float(qo + lse), "mlp": float(gu), "total": float(qo + lse + gu)}


def tpsp_layouts(devices: int):
    """Every T x Sigma = devices layout with both degrees above 1 or T = 1."""
    return [Layout("tpsp", t, devices // t) for t in range(1, devices) if devices % t == 0]


def report(model: Model = MODEL_7B, pages: dict = PAGES_128K, seqs=(4096, 32768, 131072)) -> str:
    """Per-GPU GB of each layout at several context lengths, with the pages'
    128K figures beside the calculator's."""
    a_rep, a_sh = fit_activation_coeffs(model, pages)
    fp_rep, fp_sh = first_principles_coeffs(model)
    n = pages["devices"]
    layouts = [Layout("tsp", n), Layout("tp", n)] + tpsp_layouts(n)
    lines = [f"activation bytes per token per layer: fitted a_rep = {a_rep:.0f} ({a_rep / model.hidden:.2f} h), "
             f"a_sh = {a_sh:.0f} ({a_sh / model.hidden:.2f} h); first principles (no recomputation) "
             f"{fp_rep:.0f} / {fp_sh:.0f}",
             "layout        " + "".join(f"{f'S={s}':>12}" for s in seqs) + "   pages @128K (partly pinned)"]
    for lay in layouts:
        name = {"tsp": f"TSP D={lay.degree}", "tp": f"TP T={lay.degree}"}.get(
            lay.kind, f"TPxSP {lay.degree}x{lay.sp}")
        vals = [per_gpu_bytes(lay, model, s, 1, a_rep, a_sh)["total"] / GB for s in seqs]
        page = {"tsp": f"{pages['tsp']:.1f}", "tp": f"{pages['tp']:.1f}"}.get(
            lay.kind, f"{pages['tpsp'][0]:.1f}-{pages['tpsp'][1]:.1f} (range)")
        lines.append(f"{name:<14}" + "".join(f"{v:>12.1f}" for v in vals) + f"   {page}")
    return "\n".join(lines)


if __name__ == "__main__":
    print(report())
