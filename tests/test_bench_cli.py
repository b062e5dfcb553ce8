"""The benchmark's command-line contract that needs no GPU: it measures one GPU
only and refuses --gpus N for N > 1 with a message and a non-zero exit."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_decode_work_counts_the_index_stream():
    # 64 sequences x 262144 tokens: the bf16 idx-K stream of the 2047 competitor
    # blocks per sequence is 64 * 2047 * 128 * 128 * 2 bytes
    w = bench.decode_work(64, 262144, 64, 4, 128, 128, 16)
    assert w["bytes"]["k1d_index_pool"] >= 64 * 2047 * 128 * 128 * 2
    w8 = bench.decode_work(64, 262144, 64, 4, 128, 128, 16, fp8idx=True)
    # E4M3 bytes plus one fp32 scale per token
    assert abs(w8["bytes"]["k1d_index_pool_fp8"] - 64 * 2047 * 128 * (128 + 4)
               - 64 * 4 * 2047 * 4) < 1
    assert w8["total_bytes"] < 0.6 * w["total_bytes"]
