"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

1. The attention work plan (csrc/attn_plan.h, plain integer code shared by
   the kernels and the host) through tests/attn_plan_check.cpp, built with
   g++ -fsanitize=address,undefined.
2. The C ABI (csrc/tsp_abi.cpp: argument checks, workspace sizing, dispatch)
   built with hipcc, the sanitizers on its host side only, the kernel launchers
   replaced by host stand-ins (tests/abi_sanitize_stubs.cpp), driven through
   every entry point by tests/abi_sanitize_main.cpp.
No GPU code runs.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "folded_tensor_sequence_amd", "csrc")
TESTS = os.path.dirname(os.path.abspath(__file__))
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


def test_attention_plan_under_sanitizers(tmp_path):
    if shutil.which("g++") is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "plan_check")
    _run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
          "-fno-sanitize-recover=undefined", "-DTSP_HD=", "-I", CSRC, os.path.join(TESTS, "attn_plan_check.cpp"),
          "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert r.stdout.startswith("ok") and "runtime error" not in r.stderr


def test_c_abi_under_sanitizers(tmp_path):
    import torch
    if torch.cuda.is_available():
        pytest.skip("runs the host code against stand-in launchers on a machine without a GPU")
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path / "abi_sanitize")
    # -Xarch_host keeps the sanitizers on the host side of the hipcc line
    _run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
          "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
          "-Xarch_host", "-fno-sanitize-recover=undefined",
          "-I", os.path.join(ROOT, "include"), "-I", CSRC,
          os.path.join(CSRC, "tsp_abi.cpp"), os.path.join(TESTS, "abi_sanitize_stubs.cpp"),
          os.path.join(TESTS, "abi_sanitize_main.cpp"), "-o", exe])
    r = _run([exe], env=ENV, timeout=600)
    assert "0 failures" in r.stdout, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
