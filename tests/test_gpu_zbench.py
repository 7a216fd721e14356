"""bench.py's output contract on the GPU: one JSON line with the metric, the
roofline of the dominant kernel and the per-step statistics (a short run,
without the CPU-oracle leg, started as a child process).  Collected after the
parity tests, so that under -x a failure here hides none of them."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("partition", ["zigzag", "striped"])
def test_bench_prints_one_json_line(partition):
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    print(f"[case] bench.py --partition {partition}", flush=True)
    out = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "3", "--warmup", "1",
                          "--no-cpu-baseline", "--partition", partition],
                         capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = [ln for ln in out.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1
    j = json.loads(lines[0])
    assert j["n_gpus"] == 1 and j["steps"] == 3 and j["warmup"] == 1 and j["higher_is_better"] is True
    assert j["unit"] == "TFLOP/s" and j["value"] > 0 and j["ms_per_step"] > 0
    assert j["config"]["workload"] == "llama7b_s8k_d8" and j["config"]["partition"] == partition
    # value is the algorithmic work over the mean step time
    assert abs(j["value"] - j["gflop_per_step"] / j["ms_per_step"]) <= 1e-2 * j["value"]
    assert 0 < j["step_ms"]["min"] <= j["step_ms"]["median"]
    r = j["roofline"]
    assert r["bound"] in ("mfma", "hbm") and r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["launches"] == 3
    assert set(j["kernels_ms"]) == {"qkv", "attn", "oproj", "gateup", "down"}
    assert j["seeds"]["inputs"] == 2 and j["host"]["cores"] >= 1
    assert j["versions"]["torch"] and len(j["versions"]["libtsp_sources_sha256"]) == 16
    assert j["parity"] is None            # the oracle legs are off in this short run
    b = j["mlp_ring_bwd"]
    assert b["ms_per_call"] > 0 and b["calls"] >= 3 and b["gflop_algorithmic"] > 0
    assert abs(b["tflops"] - b["gflop_algorithmic"] / b["ms_per_call"]) <= 1e-2 * b["tflops"]
