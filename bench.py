#!/usr/bin/env python3
"""Benchmark of the MSA forward pass on one MI355X.

One step = one full pass of the hot path over one batch of seeded synthetic
input already resident in HBM: for prefill workloads a whole ``msa_prefill``
(index score + block max-pool, exp-free top-k, scheduling, KV-outer attention,
combine); for the decode workloads one ``msa_decode`` (or ``msa_decode_paged``)
over all sequences.

Prints ONE JSON line with the throughput, the roofline position of the kernel
that dominates the step (its per-launch duration measured in-process with HIP
events recorded on the library's stream), and the CPU oracle timed on a bounded
sample of the same workload as a reported baseline.  With the default workload
(prefill, L = 131072) the line also reports, under "also", the 1M-token prefill
with hot blocks and the decode step over 64 x 262144 cached tokens, each timed in
the same run with its own roofline and kernel breakdown.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--no-also]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

METRIC = "MSA prefill tokens/s @128K & 1M (1 GPU, % MFMA peak); decode us/step @256K"
DEFAULT_WORKLOAD = "prefill_L131072"
# reported beside the default workload: (workload, timed steps, warm-up steps) -- the
# other configurations of the metric (1M-token prefill with hot blocks, decode over
# 64 x 262144 cached tokens), the L = 4096 and L = 32768 prefills, decode over an
# E4M3 index-key cache and over shuffled 128-token pages, and a packed prefill of 256
# prompts of 512 tokens (sequences of at most k blocks: the dense main branch)
# (sub-millisecond steps are timed over more steps, so that one slow step -- a host
# hiccup between launches -- moves the mean little)
ALSO_WORKLOADS = (("prefill_L1048576_hot", 3, 1), ("decode_N64_L262144", 50, 5),
                  ("tiny_prefill_L4096", 50, 5), ("prefill_L32768", 10, 3),
                  ("decode_fp8idx_N64_L262144", 50, 5), ("decode_paged_N64_L262144", 50, 5),
                  ("prefill_varlen_256x512", 20, 5))
PEAK_BF16_FLOPS = 2.5e15     # MI355X dense bf16 MFMA
PEAK_HBM_BYTES = 8.0e12      # MI355X HBM3E
B_BLOCK = 128
K4_QUERIES = 128             # (query, slot) entries per KV-outer work item

# The roofline that bounds each kernel: the two contractions (index scores, sparse
# attention) on the bf16 matrix cores, measured by their algorithmic FLOPs; every
# other kernel on HBM bandwidth, measured by its algorithmic bytes.
KERNEL_ROOF = {
    "k1_index_pool": "mfma", "k12_index_select": "mfma", "k4_kv_outer": "mfma",
    "k2_select": "hbm", "k3_schedule": "hbm", "k5_combine": "hbm",
    "k1d_index_pool": "hbm", "k1d_index_pool_fp8": "hbm", "k4d_merge": "hbm",
    "k4d_split": "hbm", "k4d_online": "hbm", "k4d_parts": "hbm", "page_check": "hbm",
    "quantize_e4m3": "hbm", "kd_dense": "mfma",
}


# --------------------------------------------------------------------------
# Algorithmic work model
# --------------------------------------------------------------------------
def paper_flop_ratio(H: int, G: int, d: int, dI: int, L: int, kB: int) -> float:
    """Per-token attention FLOPs of dense causal GQA over MSA (index branch plus
    main branch), averaged over a causal sequence of L tokens."""
    dense = 4 * H * d * (L / 2)
    msa = 4 * H * d * kB + 2 * G * dI * (L / 2)
    return dense / msa


K12_MIN_WORKGROUPS = 1024          # the library's floor for a fused launch
K12_QUERY_BLOCK_PARTS = {1: 1, 2: 2, 4: 2, 8: 4}   # K12 work-groups per query block


def fused_index_rows(L, k, chunk=131072, B=B_BLOCK, G=4):
    """Query rows whose index branch the fused kernel (k12_index_select) serves: those
    of query chunks whose shortest row has at least as many competitor blocks as the
    chunk has query blocks and that give the kernel at least 1024 work-groups (the
    library's rule; chunks of `chunk` queries from 0)."""
    fused = np.zeros(L, bool)
    if k - 1 > 16:
        return fused
    for q0 in range(0, L, chunk):
        qend = min(L, q0 + chunk)
        nqb = -(-(qend - q0) // B)
        if q0 // B >= nqb and nqb * K12_QUERY_BLOCK_PARTS[G] >= K12_MIN_WORKGROUPS:
            fused[q0:qend] = True
    return fused


def prefill_work(L, H, G, d, dI, k, B=B_BLOCK, list_counts=None, chunk=131072, dense_main=True):
    """Algorithmic FLOPs and bytes of each prefill kernel over one whole step.

    K1 scores every competitor key of every (query, group): 2*G*dI FLOP per
    (query, key) pair with key block < b(i).  K4 attends, per (query, group),
    the tokens of its selected blocks inside the causal window: 4*r*d FLOP per
    attended (query, group, token) for the r heads of the group.  Those two are
    measured by FLOPs; the bytes they move are the design's (the block-score hand-off
    from K1 to K2; K4's gathered q rows, partial rows and staged K/V blocks) and are
    reported apart, under "design_bytes".  The HBM-bound kernels K2, K3 and K5 are
    measured by their bytes.

    A sequence of at most k blocks selects every causal block of every query
    whatever the scores, so the library runs its main branch as dense causal
    attention (kd_dense) without the index branch: its work is the attention's
    4*r*d FLOP per (query, group, causal key), and no index FLOPs.  The call on
    given ids (dense_main=False) always runs the KV-outer kernels.
    """
    r = H // G
    i = np.arange(L, dtype=np.int64)
    bi = i // B
    nsel = np.minimum(k, bi + 1)
    pairs = float(np.sum(bi * B))                                     # scored (query, key)
    attended = float(np.sum((nsel - 1) * B + (i - bi * B + 1)))       # per group
    dense_gqa = 4.0 * H * d * float(np.sum(i + 1))
    if dense_main and L <= k * B:
        tile = 4 * (32 // r)                      # queries per kd_dense work-group
        tiles = -(-L // tile)
        staged = sum(((t * tile) // B + 1) for t in range(tiles)) * G * 2 * B * d * 2.0
        return {
            "flops": {"kd_dense": dense_gqa},
            "bytes": {},
            "design_bytes": {"kd_dense": {"q_in": L * H * d * 2.0, "out": L * H * d * 2.0,
                                          "ids_out": 4.0 * L * G * k,
                                          "kv_blocks_staged": staged}},
            "pairs": 0.0, "attended_per_group": attended, "entries": float(np.sum(nsel)) * G,
            "f_total": dense_gqa, "dense_gqa_flops": dense_gqa,
        }
    entries = float(np.sum(nsel)) * G                                 # (query, group, slot)
    f_idx = 2.0 * G * dI * pairs
    fused = fused_index_rows(L, k, chunk, B, G)
    f_k12 = 2.0 * G * dI * float(np.sum((bi * B)[fused]))
    f_attn = 4.0 * r * d * G * attended
    items = float(np.sum(np.ceil(np.asarray(list_counts) / K4_QUERIES))) \
        if list_counts is not None else entries / K4_QUERIES
    k5_bytes = entries * r * (2 * d + 4) + L * H * d * 2 + 4.0 * L * G * k
    unf = ~fused
    k2_bytes = (4.0 * G * float(np.sum(np.where((bi > k - 1) & unf, bi, 0)))
                + 4.0 * float(np.sum(unf)) * G * k)
    return {
        "flops": {"k1_index_pool": f_idx - f_k12, "k12_index_select": f_k12,
                  "k4_kv_outer": f_attn},
        "bytes": {"k2_select": k2_bytes, "k3_schedule": 12.0 * L * G * k,
                  "k5_combine": k5_bytes},
        "design_bytes": {
            "k1_index_pool": {"idx_q_in": float(np.sum(unf)) * G * dI * 2.0,
                              "block_scores_out": 4.0 * G * float(np.sum(bi[unf]))},
            "k12_index_select": {"idx_q_in": float(np.sum(fused)) * G * dI * 2.0,
                                 "ids_out": 4.0 * float(np.sum(fused)) * G * k},
            "k4_kv_outer": {"q_rows_gathered": entries * r * d * 2.0,
                            "partial_rows_out": entries * r * (2 * d + 4.0),
                            "kv_blocks_staged": items * 2 * B * d * 2.0}},
        "pairs": pairs, "attended_per_group": attended, "entries": entries,
        "f_total": f_idx + f_attn,
        "dense_gqa_flops": dense_gqa,
    }


def decode_work(N, Lc, H, G, d, dI, k, B=B_BLOCK, paged=False, fp8idx=False):
    p = Lc - 1
    nb = p // B                                        # competitor blocks per sequence
    nsel = min(k, nb + 1)
    # idx-K cache stream: bf16, or E4M3 bytes plus one fp32 scale per token
    idx_bytes = N * nb * B * (dI + 4.0 if fp8idx else dI * 2.0)
    kv_bytes = N * G * nsel * 2 * B * d * 2.0          # selected K and V blocks
    small = N * (H * d * 2 * 2 + G * dI * 2) + N * G * (nb * 4 * 2 + k * 4)
    if paged:                                          # block-table reads
        small += N * (nb + 1) * 4.0 * 2 + N * G * nsel * 4.0 * 2
    part = N * H * nsel * (2 * d + 4) * 2.0
    # parts per (sequence, group) of the decode attention (the library's rule: one
    # launch from 256 (sequence, group) pairs on, else parts for 512 work-groups);
    # with parts, K5 merges P partials per head
    P = 1 if N * G >= 256 else min(k, -(-512 // (N * G)))
    k1d = "k1d_index_pool_fp8" if fp8idx else "k1d_index_pool"
    return {
        "bytes": {k1d: idx_bytes + N * G * nb * 4.0,
                  "k4d_split": kv_bytes + N * H * nsel * (d * 2 + 2 * d + 4),
                  "k2_select": N * G * (nb * 4.0 + k * 4),
                  "k5_combine": (N * H * min(P, nsel) * (2 * d + 4) if P > 1 else part / 2)
                  + N * H * d * 2,
                  # the one-launch forms: K/V and q in, the output out, partials stay on chip
                  "k4d_merge": kv_bytes + N * H * d * 2 * 2,
                  "k4d_online": kv_bytes + N * H * d * 2 * 2,
                  # in parts: K/V and q in, one normalised partial per (head, part) out
                  "k4d_parts": kv_bytes + N * H * d * 2 + N * H * min(P, nsel) * (2 * d + 4)},
        "total_bytes": idx_bytes + kv_bytes + small + part,
        "flops": 2.0 * N * G * dI * nb * B + 4.0 * N * H * d * ((nsel - 1) * B + (p % B) + 1),
    }


def _add_work(a, b):
    """Sum of two prefill_work records (work of a batch of sequences)."""
    out = {}
    for key, val in a.items():
        out[key] = _add_work(val, b[key]) if isinstance(val, dict) else val + b[key]
    return out


def roofline(kernel: str, work: dict, n_launch: float, avg_launch_ms: float) -> dict:
    """Roofline position of one kernel: its algorithmic work per launch (FLOPs for the
    matrix-core kernels, bytes for the others, per KERNEL_ROOF) over its average launch
    duration, against MI355X's published peak.  For a matrix-core kernel the bytes its
    design moves are reported beside it (design_bytes_per_launch), never as its work."""
    t = avg_launch_ms / 1e3
    if KERNEL_ROOF[kernel] == "mfma":
        f = work["flops"][kernel] / n_launch
        roof = {"bound": "mfma", "achieved": f / t / 1e12, "peak": PEAK_BF16_FLOPS / 1e12,
                "unit": "TFLOP/s", "flops_per_launch": f}
        design = work.get("design_bytes", {}).get(kernel)
        if design:
            per = {name: v / n_launch for name, v in design.items()}
            roof["design_bytes_per_launch"] = per
            roof["design_bytes_GBps"] = sum(per.values()) / t / 1e9
    else:
        b = work["bytes"][kernel] / n_launch
        roof = {"bound": "hbm", "achieved": b / t / 1e9, "peak": PEAK_HBM_BYTES / 1e9,
                "unit": "GB/s", "bytes_per_launch": b}
    roof["frac"] = roof["achieved"] / roof["peak"]
    return roof


# --------------------------------------------------------------------------
def _host():
    """What the CPU baseline ran on: visible cores and the CPU model."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu_model": model,
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _sample_rows(L, n, seed=0):
    rng = np.random.default_rng(seed)
    return np.sort(rng.choice(L, size=min(n, L), replace=False))


def cpu_baseline_prefill(x, shape, target_s=15.0):
    """Time the oracle on a random sample of query rows of the same workload."""
    import oracle
    lib = oracle.load()
    host = {n: x[n].cpu() for n in ("q", "k", "v", "iq", "ik")}
    scale = 1.0 / math.sqrt(shape.d)
    n = 16
    total_rows, total_s = 0, 0.0
    seed = 1
    while total_s < target_s:
        rows = _sample_rows(shape.L, n, seed)
        t0 = time.perf_counter()
        oracle.prefill(host["q"], host["k"], host["v"], host["iq"], host["ik"], B_BLOCK, shape.k,
                       scale, rows=rows, lib=lib)
        dt = time.perf_counter() - t0
        total_rows += len(rows)
        total_s += dt
        seed += 1
        if dt < target_s / 8:
            n *= 2
    return {"value": total_rows / total_s, "unit": "tokens/s",
            "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"{total_rows} query rows drawn uniformly from the L={shape.L} workload "
                      f"(each row: index scores vs all causal keys, selection, attention over "
                      f"its blocks), {total_s:.1f} s wall"}


def cpu_baseline_sparse_attn(x, ids, shape, target_s=15.0):
    """The oracle's main branch on a random sample of query rows, given the same ids."""
    import oracle
    lib = oracle.load()
    host = {n: x[n].cpu() for n in ("q", "k", "v")}
    ids_h = ids.cpu().numpy()
    scale = 1.0 / math.sqrt(shape.d)
    n, seed = 64, 1
    total_rows, total_s = 0, 0.0
    while total_s < target_s:
        rows = _sample_rows(shape.L, n, seed)
        t0 = time.perf_counter()
        oracle.attend(host["q"], host["k"], host["v"], ids_h[rows], B_BLOCK, scale, rows=rows,
                      lib=lib)
        dt = time.perf_counter() - t0
        total_rows += len(rows)
        total_s += dt
        seed += 1
        if dt < target_s / 8:
            n *= 2
    return {"value": total_rows / total_s, "unit": "tokens/s",
            "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"{total_rows} query rows drawn uniformly from the L={shape.L} workload "
                      f"(each row: attention of all heads over its listed blocks), "
                      f"{total_s:.1f} s wall"}


def cpu_baseline_decode(x, shape, target_s=15.0):
    """The decode oracle on batches of whole sequences (E4M3 index-key variant when
    the workload's index cache is FP8)."""
    import oracle
    lib = oracle.load()
    fp8 = "ik8" in x
    t_copy = time.perf_counter()
    n_seq = 1
    host = None
    total, total_s = 0, 0.0
    while total_s < target_s and total < shape.N:
        seqs = np.arange(total, min(shape.N, total + n_seq))
        if host is None:
            host = {n: x[n].cpu() for n in ("q", "iq")}
        sl = slice(seqs[0], seqs[-1] + 1)
        kc = x["k_cache"][sl].cpu()
        vc = x["v_cache"][sl].cpu()
        if fp8:
            ik8, iks = x["ik8"][sl].cpu(), x["ik_scale"][sl].cpu()
        else:
            ikc = x["ik_cache"][sl].cpu()
        t0 = time.perf_counter()
        if fp8:
            oracle.decode_fp8idx(host["q"][sl], host["iq"][sl], kc, vc, ik8, iks,
                                 np.asarray(x["seq_len"])[seqs], B_BLOCK, shape.k, lib=lib)
        else:
            oracle.decode(host["q"][sl], host["iq"][sl], kc, vc, ikc,
                          np.asarray(x["seq_len"])[seqs], B_BLOCK, shape.k, lib=lib)
        total_s += time.perf_counter() - t0
        total += len(seqs)
        n_seq = min(16, n_seq * 2)
    us_per_step = total_s / total * shape.N * 1e6
    del t_copy
    return {"value": us_per_step, "unit": "us/step", "cores": oracle.num_threads(lib),
            "kind": "oracle",
            "sample": f"{total} of {shape.N} sequences ({total_s:.1f} s wall), scaled to all "
                      f"{shape.N}"}


def cpu_baseline_decode_paged(x, shape, target_s=15.0):
    """The paged oracle on batches of whole sequences: the pages a batch's tables
    name are copied to the host; the oracle gathers them and decodes the batch."""
    import oracle
    lib = oracle.load()
    q, iq = x["q"].cpu(), x["iq"].cpu()
    table = x["block_table"]
    lens = np.asarray(x["seq_len"], np.int64)
    total, total_s, n_seq = 0, 0.0, 1
    while total_s < target_s and total < shape.N:
        seqs = np.arange(total, min(shape.N, total + n_seq))
        pages = table[seqs[0]:seqs[-1] + 1].long()
        local = np.arange(pages.numel(), dtype=np.int32).reshape(pages.shape)
        sl = slice(seqs[0], seqs[-1] + 1)
        if "ik8_pages" in x:
            kp, vp, ik8p, kscp = (x[name][pages.reshape(-1)].cpu() for name in
                                  ("k_pages", "v_pages", "ik8_pages", "ik_scale_pages"))
            t0 = time.perf_counter()
            oracle.decode_paged_fp8idx(q[sl], iq[sl], kp, vp, ik8p, kscp, local, lens[seqs],
                                       B_BLOCK, shape.k, lib=lib)
        else:
            kp, vp, ikp = (x[name][pages.reshape(-1)].cpu()
                           for name in ("k_pages", "v_pages", "ik_pages"))
            t0 = time.perf_counter()
            oracle.decode_paged(q[sl], iq[sl], kp, vp, ikp, local, lens[seqs], B_BLOCK, shape.k,
                                lib=lib)
        total_s += time.perf_counter() - t0
        total += len(seqs)
        n_seq = min(16, n_seq * 2)
    return {"value": total_s / total * shape.N * 1e6, "unit": "us/step",
            "cores": oracle.num_threads(lib), "kind": "oracle",
            "sample": f"{total} of {shape.N} sequences ({total_s:.1f} s wall, page gather "
                      f"included), scaled to all {shape.N}"}


def dense_gqa_baseline(x, shape, msa_ms, reps=3):
    """Dense causal GQA attention on the same q/k/v with PyTorch's fused SDPA
    backends (flash / memory-efficient; the math backend is never allowed, it would
    materialise L x L).  A library timing for the sparse-vs-dense comparison."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel
    r = shape.H // shape.G
    q = x["q"].transpose(0, 1).unsqueeze(0).contiguous()                  # [1, H, L, d]
    k = x["k"].transpose(0, 1).repeat_interleave(r, dim=0).unsqueeze(0).contiguous()
    v = x["v"].transpose(0, 1).repeat_interleave(r, dim=0).unsqueeze(0).contiguous()
    res = {"backend": None, "ms": None, "tflops": None, "speedup_msa_vs_dense": None}
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION),
                     ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            with sdpa_kernel([be]):
                torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
                e1.record()
                torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            flops = 4.0 * shape.H * shape.d * shape.L * (shape.L + 1) / 2
            res.update({"backend": name, "ms": ms, "tflops": flops / (ms / 1e3) / 1e12,
                        "speedup_msa_vs_dense": ms / msa_ms})
            break
        except RuntimeError as e:            # backend not available for this shape
            res["error_" + name] = str(e).splitlines()[0][:160]
    del q, k, v
    torch.cuda.empty_cache()
    return res


def copy_calibration(gib: float):
    """A plain copy of known size: each launch reads and writes exactly n bytes."""
    import torch
    n = int(gib * (1 << 30)) // 16 * 16
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 4}), flush=True)


def gemm_reference(n=8192, reps=20):
    """What a plain library bf16 GEMM (torch.matmul -> hipBLASLt) sustains on this GPU,
    on N(0,1) operands and on constant ones: the practical matrix-core rate the
    contraction kernels are compared with, and how much the operand values alone
    move it (a power-limited clock)."""
    import torch
    res = {"shape": [n, n, n], "dtype": "bf16", "library": "torch.matmul (hipBLASLt)"}
    g = torch.Generator(device="cuda:0")
    g.manual_seed(0)
    for name in ("random", "constant"):
        if name == "random":
            a = torch.randn((n, n), generator=g, device="cuda:0").to(torch.bfloat16)
            b = torch.randn((n, n), generator=g, device="cuda:0").to(torch.bfloat16)
        else:
            a = torch.full((n, n), 1.0, device="cuda:0", dtype=torch.bfloat16)
            b = torch.full((n, n), 1.0, device="cuda:0", dtype=torch.bfloat16)
        c = torch.empty((n, n), device="cuda:0", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        res[name + "_tflops"] = 2.0 * n ** 3 / (ms / 1e3) / 1e12
        del a, b, c
    res["random_frac_of_peak"] = res["random_tflops"] * 1e12 / PEAK_BF16_FLOPS
    return res


def sources_code_hash(paths) -> str:
    """First 16 hex digits of the SHA-256 of the given source files' code: comments
    removed and every run of whitespace made one space, so that a change to the
    comments alone leaves a counter record valid and any change to the code does
    not."""
    import hashlib
    h = hashlib.sha256()
    for fp in paths:
        text = open(fp, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def _load_traffic(kernel: str, workload: str):
    """HBM traffic per launch from a committed rocprofv3 counter summary, if one is
    recorded for this kernel and workload and the source files it names (those
    that decide the kernel's code, launch and work list) are unchanged."""
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.strip().startswith("-"):
            key, _, val = line.strip("- \n").partition(":")
            rec[key.strip()] = val.strip()
    files = rec.get("sources", "").split()
    if not files:
        return None
    src = os.path.join(here, "block_sparse_long_idx_amd", "csrc")
    paths = [os.path.join(src, f) for f in files]
    if not all(os.path.exists(fp) for fp in paths):
        return None
    if rec.get("sources_sha256_16") != sources_code_hash(paths):
        return None
    try:
        return float(rec["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_workload(args, name, steps, warmup, cpu_baseline, dense):
    """Warm up, time exactly `steps` steps of one workload, break them down per
    kernel, and return the result record (roofline, optional CPU and dense
    baselines)."""
    import torch
    import block_sparse_long_idx_amd as msa
    import synth

    wl = synth.WORKLOADS[name]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] workload {wl.name}: generating inputs on {dev}", file=sys.stderr, flush=True)
    s = wl.shape

    if wl.kind == "prefill":
        x = synth.prefill_inputs(s, seed=args.seed, plant=wl.plant, n_plant=wl.n_plant, c=wl.c,
                                 hot_blocks=wl.hot_blocks, device=dev)
        out = torch.empty_like(x["q"])
        ids = torch.empty((s.L, s.G, s.k), dtype=torch.int32, device=dev)
        ws = msa._workspace(msa.workspace_size("prefill", L=s.L, H=s.H, G=s.G, d=s.d, dI=s.dI,
                                               k=s.k), dev)

        def step():
            msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=s.k, out=out,
                        ids_out=ids, workspace=ws, return_ids=True)
    elif wl.kind == "sparse_attn":     # main branch alone on constructed skewed ids
        x = synth.prefill_inputs(s, seed=args.seed, plant="none", device=dev)
        ids = synth.skewed_ids(s.L, s.G, s.k, hot=wl.hot_blocks, seed=args.seed, device=dev)
        out = torch.empty_like(x["q"])
        ws = msa._workspace(msa.workspace_size("sparse_attn", L=s.L, H=s.H, G=s.G, d=s.d,
                                               k=s.k), dev)

        def step():
            msa.sparse_attn(x["q"], x["k"], x["v"], ids, out=out, workspace=ws)
    elif wl.kind == "prefill_varlen":
        parts = [synth.prefill_inputs(s, seed=args.seed + b, plant=wl.plant, n_plant=wl.n_plant,
                                      c=wl.c, device=dev) for b in range(wl.batch)]
        x = {n: torch.cat([p_[n] for p_ in parts]) for n in ("q", "k", "v", "iq", "ik")}
        del parts
        T = wl.batch * s.L
        out = torch.empty_like(x["q"])
        ids = torch.empty((T, s.G, s.k), dtype=torch.int32, device=dev)
        cu_all = [b * s.L for b in range(wl.batch + 1)]
        ws = msa._workspace(msa.workspace_size("prefill_varlen", cu_q=cu_all, cu_kv=cu_all, H=s.H,
                                               G=s.G, d=s.d, dI=s.dI, k=s.k), dev)
        if wl.chunk:       # one sequence, `chunk` new tokens per call over the cached prefix
            calls = []
            for P in range(0, s.L, wl.chunk):
                C = min(wl.chunk, s.L - P)
                calls.append((x["q"][P:P + C], x["iq"][P:P + C], x["k"][:P + C], x["v"][:P + C],
                              x["ik"][:P + C], [0, C], [0, P + C], out[P:P + C], ids[P:P + C]))
        else:              # the whole batch in one call
            cu = [b * s.L for b in range(wl.batch + 1)]
            calls = [(x["q"], x["iq"], x["k"], x["v"], x["ik"], cu, cu, out, ids)]

        def step():
            for qq, iqq, kk, vv, ikk, cq, ckv, oo, ii in calls:
                msa.prefill_varlen(qq, kk, vv, iqq, ikk, cq, ckv, kslots=s.k, out=oo, ids_out=ii,
                                   workspace=ws, return_ids=True)
    elif wl.kind == "decode":
        x = synth.decode_inputs(s, seed=args.seed, device=dev)
        seq_len = torch.tensor(np.asarray(x["seq_len"], np.int32), device=dev)
        out = torch.empty_like(x["q"])
        ids = torch.empty((s.N, s.G, s.k), dtype=torch.int32, device=dev)
        ws = msa._workspace(msa.workspace_size("decode", N=s.N, Lmax=s.Lc, H=s.H, G=s.G, d=s.d,
                                               dI=s.dI, k=s.k), dev)

        def step():
            msa.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"], seq_len,
                       kslots=s.k, out=out, ids_out=ids, workspace=ws, return_ids=True)
    elif wl.kind == "decode_fp8idx":   # index-key cache as E4M3 bytes + per-token scales
        x = synth.decode_inputs(s, seed=args.seed, device=dev)
        x["ik8"], x["ik_scale"] = msa.quantize_idx_k_e4m3(x["ik_cache"])
        del x["ik_cache"]
        torch.cuda.empty_cache()
        seq_len = torch.tensor(np.asarray(x["seq_len"], np.int32), device=dev)
        out = torch.empty_like(x["q"])
        ids = torch.empty((s.N, s.G, s.k), dtype=torch.int32, device=dev)
        ws = msa._workspace(msa.workspace_size("decode", N=s.N, Lmax=s.Lc, H=s.H, G=s.G, d=s.d,
                                               dI=s.dI, k=s.k), dev)

        def step():
            msa.decode_fp8idx(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik8"],
                              x["ik_scale"], seq_len, kslots=s.k, out=out, ids_out=ids,
                              workspace=ws, return_ids=True)
    else:   # decode over 128-token pages in a seeded random order
        e4m3 = wl.kind == "decode_paged_fp8idx"
        x = synth.decode_inputs(s, seed=args.seed, device=dev)
        names = ("k_cache", "v_cache", "ik_cache")
        if e4m3:
            x["ik8"], x["ik_scale"] = msa.quantize_idx_k_e4m3(x["ik_cache"])
            names = ("k_cache", "v_cache", "ik8", "ik_scale")
        x.update(synth.paginate(x, B_BLOCK, seed=args.seed, names=names))
        for name in ("k_cache", "v_cache", "ik_cache", "ik8", "ik_scale"):
            x.pop(name, None)
        torch.cuda.empty_cache()
        seq_len = torch.tensor(np.asarray(x["seq_len"], np.int32), device=dev)
        out = torch.empty_like(x["q"])
        ids = torch.empty((s.N, s.G, s.k), dtype=torch.int32, device=dev)
        maxb = x["block_table"].shape[1]
        ws = msa._workspace(msa.workspace_size("decode_paged", N=s.N, max_blocks=maxb, H=s.H,
                                               G=s.G, d=s.d, dI=s.dI, k=s.k), dev)

        def step():
            if e4m3:
                msa.decode_paged_fp8idx(x["q"], x["iq"], x["k_pages"], x["v_pages"],
                                        x["ik8_pages"], x["ik_scale_pages"], x["block_table"],
                                        seq_len, kslots=s.k, out=out, ids_out=ids, workspace=ws,
                                        return_ids=True)
            else:
                msa.decode_paged(x["q"], x["iq"], x["k_pages"], x["v_pages"], x["ik_pages"],
                                 x["block_table"], seq_len, kslots=s.k, out=out, ids_out=ids,
                                 workspace=ws, return_ids=True)

    torch.cuda.synchronize()
    print(f"[bench] warmup {warmup}", file=sys.stderr, flush=True)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps --------------------------------------
    print(f"[bench] timing {steps} steps", file=sys.stderr, flush=True)
    # one event between consecutive steps: the K-step total and each step's time
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev[0].record()
    for i in range(steps):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t_wall
    ms_per_step = ev[0].elapsed_time(ev[-1]) / steps
    step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    median_ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else \
        0.5 * (step_ms[len(step_ms) // 2 - 1] + step_ms[len(step_ms) // 2])

    # ---- per-kernel breakdown: the same K steps with stage events -----------
    msa.timing_enable(64 * steps + 64)
    for _ in range(steps):
        step()
    per_kernel = msa.timing_collect()
    msa.timing_disable()
    kernels = {name: {"launches_per_step": n / steps, "ms_per_step": tot / steps,
                      "avg_launch_ms": tot / n} for name, (n, tot) in per_kernel.items()}
    dominant = max(kernels, key=lambda k_: kernels[k_]["ms_per_step"])

    result = {"metric": METRIC, "n_gpus": 1, "steps": steps, "warmup": warmup,
              "ms_per_step": ms_per_step, "ms_per_step_median": median_ms,
              "ms_per_step_min": step_ms[0], "scaling": "weak", "vs_baseline": None,
              "dtype": "bf16", "data": "synthetic (seeded N(0,1) bf16, planted blocks)"}
    if wl.kind in ("prefill", "prefill_varlen", "sparse_attn"):
        nseq = wl.batch
        idn = ids.cpu().numpy().reshape(nseq, s.L, s.G, s.k)
        work = None
        for b in range(nseq):
            valid = idn[b] >= 0
            g_idx = np.broadcast_to(np.arange(s.G)[None, :, None], idn[b].shape)
            counts = np.bincount((g_idx[valid] * ((s.L + 127) // 128) + idn[b][valid]).ravel(),
                                 minlength=s.G * ((s.L + 127) // 128))
            w_b = prefill_work(s.L, s.H, s.G, s.d, s.dI, s.k, list_counts=counts,
                               dense_main=wl.kind != "sparse_attn")
            work = w_b if work is None else _add_work(work, w_b)
        result.update({"value": nseq * s.L / (ms_per_step / 1e3), "unit": "tokens/s",
                       "higher_is_better": True})
        result["config"] = {"workload": wl.name, "L": s.L, "H": s.H, "G": s.G, "d": s.d,
                            "dI": s.dI, "B": s.B, "k": s.k, "planting": wl.plant,
                            "query_chunk": min(-(-s.L // 128) * 128, 131072)}
        if wl.kind == "prefill_varlen":
            result["config"].update({"sequences": nseq, "new_tokens_per_call": wl.chunk or s.L})
        if wl.kind == "sparse_attn":   # no index branch in the step
            result["data"] = "synthetic (seeded N(0,1) bf16 q/k/v, constructed skewed block ids)"
            result["config"].update({"ids": "constructed: blocks %s + own block + %d random"
                                            % (list(wl.hot_blocks), s.k - 1 - len(wl.hot_blocks))})
            del result["config"]["planting"]
            for key_ in ("k1_index_pool", "k12_index_select", "k2_select"):
                work["flops"].pop(key_, None)
                work["bytes"].pop(key_, None)
                work["design_bytes"].pop(key_, None)
            work["f_total"] = work["flops"]["k4_kv_outer"]
        result["step_mfma_frac"] = work["f_total"] / (ms_per_step / 1e3) / PEAK_BF16_FLOPS
        result["algorithmic_flops_per_step"] = work["f_total"]
        result["dense_gqa_flops_per_step"] = work["dense_gqa_flops"]
    else:
        work = decode_work(s.N, s.Lc, s.H, s.G, s.d, s.dI, s.k,
                           paged=wl.kind in ("decode_paged", "decode_paged_fp8idx"),
                           fp8idx=wl.kind in ("decode_fp8idx", "decode_paged_fp8idx"))
        result.update({"value": ms_per_step * 1e3, "unit": "us/step", "higher_is_better": False})
        result["config"] = {"workload": wl.name, "N": s.N, "Lc": s.Lc, "H": s.H, "G": s.G,
                            "d": s.d, "dI": s.dI, "B": s.B, "k": s.k}
        result["step_hbm_frac"] = work["total_bytes"] / (ms_per_step / 1e3) / PEAK_HBM_BYTES
        # share of the planted (relevant) blocks that the selection found
        idn = ids.cpu().numpy()
        hits = [b in idn[n, g] for n, row in enumerate(x["planted"]) for g, blk in enumerate(row)
                for b in blk]
        result["planted_block_recall"] = float(np.mean(hits)) if hits else None

    # ---- roofline of the dominant kernel -------------------------------------
    kd = kernels[dominant]
    n_launch = kd["launches_per_step"]
    roof = roofline(dominant, work, n_launch, kd["avg_launch_ms"])
    roof["traffic"] = _load_traffic(dominant, wl.name)
    roof["kernel"] = dominant
    roof["launches_per_step"] = n_launch
    roof["avg_launch_ms"] = kd["avg_launch_ms"]
    result["roofline"] = roof
    result["kernels"] = {k_: {"ms_per_step": round(v["ms_per_step"], 4),
                              "launches_per_step": v["launches_per_step"]}
                         for k_, v in kernels.items()}

    # ---- CPU oracle baseline (rank 0, N=1) ------------------------------------
    if cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        if wl.kind in ("prefill", "prefill_varlen"):
            # rows of the first sequence (every sequence has the same shape)
            x0 = {n: x[n][:s.L] for n in ("q", "k", "v", "iq", "ik")}
            result["cpu_baseline"] = cpu_baseline_prefill(x0, s, args.cpu_seconds)
        elif wl.kind == "sparse_attn":
            result["cpu_baseline"] = cpu_baseline_sparse_attn(x, ids, s, args.cpu_seconds)
        elif wl.kind in ("decode", "decode_fp8idx"):
            result["cpu_baseline"] = cpu_baseline_decode(x, s, args.cpu_seconds)
        else:
            result["cpu_baseline"] = cpu_baseline_decode_paged(x, s, args.cpu_seconds)
        result["cpu_baseline"]["host"] = _host()
    want_dense = dense == "on" or (dense == "auto" and wl.kind == "prefill" and s.L <= 131072)
    if want_dense:
        print("[bench] dense causal GQA baseline (SDPA)", file=sys.stderr, flush=True)
        result["dense_baseline"] = dense_gqa_baseline(x, s, ms_per_step)
    result["wall_s_timed_region"] = wall_s
    return result


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-also", action="store_true",
                    help="with the default workload, skip the 1M-token prefill and the decode "
                         "step that the line otherwise also reports (under \"also\")")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip timing a plain bf16 library GEMM (8192^3) on random and on "
                         "constant operands, the practical matrix-core reference")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dense-baseline", choices=["auto", "on", "off"], default="auto",
                    help="time dense causal GQA attention (PyTorch SDPA, fused backends only) on "
                         "the same q/k/v; auto = prefill workloads up to L = 131072")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--copy-calibration", type=float, default=0.0, metavar="GIB",
                    help="only run a plain device-to-device copy of GIB GiB (4 times), the "
                         "reference for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the library has no multi-GPU path); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    result = run_workload(args, args.workload, args.steps, args.warmup,
                          cpu_baseline=not args.no_cpu_baseline, dense=args.dense_baseline)
    # the other two workloads of the headline metric, measured in the same run
    if args.workload == DEFAULT_WORKLOAD and not args.no_also:
        import torch
        also = {}
        for name, steps, warmup in ALSO_WORKLOADS:
            torch.cuda.empty_cache()
            r = run_workload(args, name, steps, warmup, cpu_baseline=False, dense="off")
            also[name] = {key: r[key] for key in ("value", "unit", "higher_is_better", "steps",
                                                   "warmup", "ms_per_step", "ms_per_step_median",
                                                   "ms_per_step_min", "config", "roofline",
                                                   "kernels")}
            for key in ("step_mfma_frac", "step_hbm_frac", "planted_block_recall"):
                if key in r:
                    also[name][key] = r[key]
        result["also"] = also
    if not args.no_gemm_reference:
        result["gemm_reference"] = gemm_reference()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
