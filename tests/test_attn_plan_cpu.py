"""Host check of the attention work plan.

The plan (which rows and key tiles each attention work group computes, where
split pieces go in the workspace, how the merge finds them) is plain integer
code in ``folded_tensor_sequence_amd/csrc/attn_plan.h``, shared by the GPU
kernels and compiled here on its own with g++ together with
``tests/attn_plan_check.cpp``, which checks for thousands of rank shapes that
every (row block, sequence x q-head, key tile) is computed exactly once, both
paired and unpaired, for 128- and 256-row blocks.
"""
import pathlib
import shutil
import subprocess

import pytest

ROOT = pathlib.Path(__file__).resolve().parents[1]


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_attention_plan_covers_every_tile_once(tmp_path):
    exe = tmp_path / "attn_plan_check"
    subprocess.run(["g++", "-std=c++17", "-O2", "-DTSP_HD=", f"-I{ROOT / 'folded_tensor_sequence_amd' / 'csrc'}",
                    str(ROOT / "tests" / "attn_plan_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr
