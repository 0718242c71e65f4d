"""GPU parity through the C ABI alone: tests/bin/c_gpu_prefill (built from
tests/c_gpu_prefill.c by the package build) allocates with the HIP runtime,
runs a bf16 prefill (two sequences, three heads, 700 tokens, initial
states, segments cut at 256 tokens) and a decode step through the library's
C entry points, and compares every output and state element with the
double-precision oracle (max |x - x_ref| / max |x_ref| <= 2e-2)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "bin", "c_gpu_prefill")


def test_c_caller_prefill_and_decode():
    assert os.path.exists(BIN), "tests/bin/c_gpu_prefill is not built (run the package build)"
    print("running", BIN, flush=True)
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=300)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("PASS")
