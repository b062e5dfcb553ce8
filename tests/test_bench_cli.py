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


def test_traffic_record_follows_its_sources(tmp_path, monkeypatch):
    """A counter record counts only while the sources it names hash as recorded:
    the committed records load, and a record whose hash no longer matches (a kernel
    changed after its counters were taken) gives no traffic figure."""
    import glob
    import hashlib
    import re
    records = glob.glob(os.path.join(ROOT, "profiles", "traffic_*.md"))
    assert records
    for path in records:
        text = open(path).read()
        kernel = re.search(r"- kernel: (\S+)", text).group(1)
        workload = re.search(r"- workload: (\S+)", text).group(1)
        files = re.search(r"- sources: (.*)", text).group(1).split()
        h = hashlib.sha256()
        for f in files:
            code = open(os.path.join(ROOT, "block_sparse_long_idx_amd", "csrc", f)).read()
            # the code alone: block and line comments out, whitespace runs as one space
            code = re.sub(r"//[^\n]*", " ", re.sub(r"/\*.*?\*/", " ", code, flags=re.S))
            h.update(" ".join(code.split()).encode() + b"\0")
        current = re.search(r"- sources_sha256_16: (\w+)", text).group(1) == h.hexdigest()[:16]
        val = bench._load_traffic(kernel, workload)
        # a value exactly when the record matches the sources as they are now
        assert (val is not None) == current, (kernel, workload)
        if current:
            assert val == float(re.search(r"- hbm_bytes_per_launch: (\d+)", text).group(1))
    # a copy of the repository layout with one record whose hash is stale
    import shutil
    fake = tmp_path / "repo"
    (fake / "profiles").mkdir(parents=True)
    shutil.copytree(os.path.join(ROOT, "block_sparse_long_idx_amd", "csrc"),
                    fake / "block_sparse_long_idx_amd" / "csrc")
    src = open(os.path.join(ROOT, "profiles", "traffic_k4_kv_outer_prefill_L131072.md")).read()
    stale = re.sub(r"sources_sha256_16: \w+", "sources_sha256_16: 0000000000000000", src)
    (fake / "profiles" / "traffic_k4_kv_outer_prefill_L131072.md").write_text(stale)
    shutil.copy(os.path.join(ROOT, "bench.py"), fake / "bench.py")
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_copy", fake / "bench.py")
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    assert mod._load_traffic("k4_kv_outer", "prefill_L131072") is None
    assert mod._load_traffic("k4_kv_outer", "no_such_workload") is None
    # the record stamped with the copy's own sources: valid; still valid after a
    # comment edit to a source it names; void after a change to that source's code
    files = re.search(r"- sources: (.*)", src).group(1).split()
    h = hashlib.sha256()
    for f in files:
        code = open(fake / "block_sparse_long_idx_amd" / "csrc" / f).read()
        code = re.sub(r"//[^\n]*", " ", re.sub(r"/\*.*?\*/", " ", code, flags=re.S))
        h.update(" ".join(code.split()).encode() + b"\0")
    fresh = re.sub(r"sources_sha256_16: \w+", "sources_sha256_16: " + h.hexdigest()[:16], src)
    (fake / "profiles" / "traffic_k4_kv_outer_prefill_L131072.md").write_text(fresh)
    assert mod._load_traffic("k4_kv_outer", "prefill_L131072") is not None
    attn = fake / "block_sparse_long_idx_amd" / "csrc" / "msa_attn.hip"
    code = attn.read_text()
    attn.write_text("// a new comment line\n/* and a block\n   comment */\n" + code)
    assert mod._load_traffic("k4_kv_outer", "prefill_L131072") is not None
    attn.write_text(code.replace("kBlock", "kBlock ", 1).replace("return", "return  ", 1)
                    .replace("namespace msa {", "namespace msa {\nconstexpr int kUnused = 1;", 1))
    assert mod._load_traffic("k4_kv_outer", "prefill_L131072") is None


def test_every_workload_kind_is_benchmarked():
    import synth
    kinds = {"prefill", "prefill_varlen", "sparse_attn", "decode", "decode_fp8idx",
             "decode_paged", "decode_paged_fp8idx"}
    src = open(os.path.join(ROOT, "bench.py")).read()
    for name, wl in synth.WORKLOADS.items():
        assert wl.kind in kinds, name
        assert f'"{wl.kind}"' in src, (name, wl.kind)
    assert bench.DEFAULT_WORKLOAD in synth.WORKLOADS
    for name, steps, warmup in bench.ALSO_WORKLOADS:
        assert name in synth.WORKLOADS and steps >= 1 and warmup >= 0
