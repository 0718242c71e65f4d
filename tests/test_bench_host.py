"""Host-side checks of bench.py (no GPU): the one-GPU contract, the byte and
FLOP formulas of the roofline, and the traffic record keyed to the kernel
sources."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_and_flops():
    # 1024 bytes per token-head (q, k, v read and out written in bf16, d = 128), the final
    # states in float32 and the decays
    B, H, N, d = 1, 64, 32768, 128
    assert bench.prefill_bytes(B, H, N, d) == B * H * N * 1024 + B * H * d * d * 4 + 4 * H
    assert bench.prefill_bytes(B, H, N, d) == 2151678208
    # decode: the float32 state read and written, q, k, v and out in bf16
    assert bench.decode_bytes(128, 64, 128) == 2 * 128 * 64 * 128 * 128 * 4 + 4 * 128 * 64 * 128 * 2
    # dense blocks: 4 d (C + d) per token-head
    assert bench.prefill_flops(B, H, N, d, 128) == B * H * N * 4 * d * (128 + d)


def test_traffic_record_matches_the_sources():
    """The committed counter record is keyed to the current kernel sources, so
    the bench line's roofline carries measured traffic."""
    with open(os.path.join(ROOT, "profiles", "traffic_layer_h64_n32k.json")) as f:
        rec = json.load(f)
    if rec["source_hash"] != bench.source_hash():
        pytest.skip("the kernel sources changed since the counters were taken: the bench "
                    "line reports traffic as null until they are taken again")
    t = bench.measured_traffic("layer_h64_n32k")
    assert t is not None and t["step"] == rec["bytes_per_step"]
    # the chunk kernel moves close to its algorithmic bytes
    ratio = t["prefill_chunk_kernel"] / bench.prefill_bytes(1, 64, 32768, 128)
    assert 1.0 <= ratio < 1.05
