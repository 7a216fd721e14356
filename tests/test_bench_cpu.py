"""Host-side checks of the benchmark's work accounting (no GPU)."""
import pytest

import bench
import synth
from oracle import tsp_oracle as orc


@pytest.mark.parametrize("partition", [0, 1], ids=["zigzag", "striped"])
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_closed_form_flops_match_the_oracle_count(name, partition):
    # bench.py counts causal pairs with a closed form; the oracle sums over the
    # rank's actual positions under the partition
    import dataclasses
    d = dataclasses.replace(synth.WORKLOADS[name].dims, partition=partition)
    mine, ref = bench.layer_flops(d), orc.algorithmic_flops(d)
    for k in ref:
        assert mine[k] == ref[k], k
    assert bench.rank_kmax(d) == int(orc.local_to_global(d.seq, d.degree, d.rank, partition).max()) + 1


def test_pair_count_is_rank_independent():
    import dataclasses
    base = synth.WORKLOADS["llama7b_s8k_d8"].dims
    counts = {bench.layer_flops(dataclasses.replace(base, rank=r))["attn"] for r in range(base.degree)}
    refs = {orc.algorithmic_flops(dataclasses.replace(base, rank=r))["attn"] for r in range(base.degree)}
    assert len(counts) == 1 and counts == refs


def test_recorded_traffic_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    import json
    src = tmp_path / "k.hip"
    src.write_text("kernel v1")
    (tmp_path / "profiles").mkdir()
    rec = {"kernel": "gateup", "workload": "w", "sources": ["k.hip"], "traffic_bytes_per_launch": 123}
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    rec["sources_sha256"] = bench.source_digest(["k.hip"])
    (tmp_path / "profiles" / "traffic_gateup_w.json").write_text(json.dumps(rec))
    assert bench.recorded_traffic("w", "gateup") == 123
    assert bench.recorded_traffic("w", "qkv") is None          # no record for that kernel
    src.write_text("kernel v2")
    assert bench.recorded_traffic("w", "gateup") is None       # counters predate the change


def test_more_than_one_gpu_is_refused():
    # the library computes one rank on one GPU: any other --gpus exits with
    # status 2 and says so, before touching a GPU
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    out = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert out.returncode == 2
    assert "--gpus must be 1" in out.stderr
    assert out.stdout == ""



def test_device_peak_from_rocminfo_text(monkeypatch):
    # the peak is recomputed from the GPU agent's own CU count and clock; the
    # CPU agent (no gfx950) is skipped
    import subprocess
    text = ("Agent 1\n  Name:  AMD EPYC\n  Device Type:  CPU\n  Compute Unit:  128\n"
            "  Max Clock Freq. (MHz):  3700\n"
            "Agent 2\n  Name:  gfx950\n  Device Type:  GPU\n  Compute Unit:  256\n"
            "  Max Clock Freq. (MHz):  2400\n")

    class Out:
        stdout = text
    monkeypatch.setattr(subprocess, "run", lambda *a, **k: Out())
    assert bench.device_peak() == {"compute_units": 256, "max_clock_mhz": 2400, "bf16_tflops": 2516.6}

    def missing(*a, **k):
        raise FileNotFoundError("rocminfo")
    monkeypatch.setattr(subprocess, "run", missing)
    assert bench.device_peak() is None
