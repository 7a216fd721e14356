"""The analytic per-GPU memory calculator (TSP, TP, TP x SP) against what the
pages fix.  Partly pinned: the pages give totals only, so two activation
coefficients are fitted to two of their figures and everything else here is
a check the fit was not made to pass.  CPU only."""
import dataclasses

import pytest

from folded_tensor_sequence_amd import memory_model as mm

GB = mm.GB
P = mm.PAGES_128K


def _fit():
    return mm.fit_activation_coeffs(mm.MODEL_7B, P)


def test_model_state_is_16_bytes_per_parameter():
    # r007 "Распределенное обучение", ZeRO worked example: 7e9 x 16 B = 112 GB
    assert mm.model_state_bytes(7e9) / GB == pytest.approx(112.0)
    assert mm.model_state_bytes(175e9) / GB == pytest.approx(2800.0)


def test_tsp_scales_both_terms_by_one_over_d():
    # "How to Fold a Book": weights and tokens both sharded 1/D on one axis
    a_rep, a_sh = _fit()
    one = mm.per_gpu_bytes(mm.Layout("tsp", 1), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)
    for d in (2, 4, 8, 16):
        got = mm.per_gpu_bytes(mm.Layout("tsp", d), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)
        assert got["model_state"] == pytest.approx(one["model_state"] / d)
        assert got["activations"] == pytest.approx(one["activations"] / d)
    # TP divides the model state the same way but keeps the replicated part
    tp = mm.per_gpu_bytes(mm.Layout("tp", 8), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)
    tsp = mm.per_gpu_bytes(mm.Layout("tsp", 8), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)
    assert tp["model_state"] == pytest.approx(tsp["model_state"])
    assert tp["activations"] > tsp["activations"]


def test_fit_reproduces_the_two_anchor_figures():
    # construction check (these two figures are what the coefficients are fitted to)
    a_rep, a_sh = _fit()
    assert a_rep > 0 and a_sh > 0
    tsp = mm.per_gpu_bytes(mm.Layout("tsp", 8), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)["total"] / GB
    tp = mm.per_gpu_bytes(mm.Layout("tp", 8), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)["total"] / GB
    assert tsp == pytest.approx(38.8) and tp == pytest.approx(70.0)


def test_predicts_the_tp_sp_range_not_fitted():
    # "What you need to know": TP+SP layouts on the same node need 85.0-140.0
    # GB; the 2x4 and 1x8 layouts (weights replicated over 4 and 8 sequence
    # shards) land on the two ends within 3%, without being fitted to them
    a_rep, a_sh = _fit()
    lo = mm.per_gpu_bytes(mm.Layout("tpsp", 2, 4), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)["total"] / GB
    hi = mm.per_gpu_bytes(mm.Layout("tpsp", 1, 8), mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)["total"] / GB
    assert lo == pytest.approx(P["tpsp"][0], rel=0.03)
    assert hi == pytest.approx(P["tpsp"][1], rel=0.03)


def test_tsp_and_tp_about_equal_at_short_context():
    # "Memory and Processing Results": model state dominates at short context
    a_rep, a_sh = _fit()
    for seq in (2048, 4096):
        tsp = mm.per_gpu_bytes(mm.Layout("tsp", 8), mm.MODEL_7B, seq, 1, a_rep, a_sh)["total"]
        tp = mm.per_gpu_bytes(mm.Layout("tp", 8), mm.MODEL_7B, seq, 1, a_rep, a_sh)["total"]
        assert tsp <= tp <= 1.10 * tsp


def test_ordering_at_128k():
    # TSP lowest at every point; TP below the weight-replicating TP+SP layouts
    a_rep, a_sh = _fit()
    tot = lambda lay: mm.per_gpu_bytes(lay, mm.MODEL_7B, P["seq"], 1, a_rep, a_sh)["total"]
    tsp, tp = tot(mm.Layout("tsp", 8)), tot(mm.Layout("tp", 8))
    assert tsp < tp < tot(mm.Layout("tpsp", 2, 4)) < tot(mm.Layout("tpsp", 1, 8))
    for lay in mm.tpsp_layouts(8):
        assert tsp < tot(lay)
    # and TSP stays the lowest at every context length
    for seq in (1024, 8192, 65536, 262144):
        t = lambda lay: mm.per_gpu_bytes(lay, mm.MODEL_7B, seq, 1, a_rep, a_sh)["total"]
        assert all(t(mm.Layout("tsp", 8)) <= t(lay) for lay in [mm.Layout("tp", 8)] + mm.tpsp_layouts(8))


def test_fitted_replicated_part_is_one_bf16_hidden_vector():
    # the fit's replicated part comes out at ~2 h bytes: one 16-bit copy of
    # the layer's input per token, which every TP rank holds in full
    a_rep, _ = _fit()
    assert a_rep == pytest.approx(2 * mm.MODEL_7B.hidden, rel=0.05)


def test_first_principles_count():
    # x and h replicated; Q, K, V, O (4 h for MHA) and gate/up/act (3 x 4 h) split
    rep, sh = mm.first_principles_coeffs(mm.MODEL_7B)
    h = mm.MODEL_7B.hidden
    assert rep == 2 * h * 2 and sh == (4 * h + 12 * h) * 2
    ungated = dataclasses.replace(mm.MODEL_7B, gated=False)
    assert mm.first_principles_coeffs(ungated)[1] == (4 * h + 8 * h) * 2
    # saving everything without recomputation needs more than the pages' TSP figure
    tsp = mm.per_gpu_bytes(mm.Layout("tsp", 8), mm.MODEL_7B, P["seq"], 1, rep, sh)["total"] / GB
    assert tsp > P["tsp"]


def test_report_prints_the_pages_figures_beside():
    text = mm.report()
    assert "38.8" in text and "70.0" in text and "85.0-140.0" in text and "partly pinned" in text
