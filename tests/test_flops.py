"""Accounting pins (CPU): the FLOP model the benchmark reports against.

"MiniMax M3 算力省 20 倍" §四 (and "MiniMax-M3上架DEVUP…") quote 28.4x fewer
attention FLOPs per token at 1M context for the 109B research model (64 query
heads, 4 KV heads, k*B = 2048).  Dense causal GQA spends 4*H*d*(L/2) per token on
average; MSA spends 4*H*d*kB on the main branch plus 2*G*dI*(L/2) on index
scores.  With dI = d the ratio is 28.44 for any d, which is the quoted figure.
"""
import numpy as np

import bench


def _page_figures():
    """tests/golden/page_figures.txt: name -> value (figures the pages print)."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "page_figures.txt")
    out = {}
    for line in open(path, encoding="utf-8"):
        if line.strip() and not line.startswith("#"):
            name, value, _src = (f.strip() for f in line.split("|", 2))
            out[name] = float(value)
    return out


def test_page_figures_reproduced():
    """The accounting and the workload shapes against the figures the pages print
    (tests/golden/page_figures.txt): the FLOP ratio at their context length and head
    counts, to the printed precision; k blocks of B tokens = the per-query key budget;
    the large workloads use the research model's heads, blocks and k."""
    import synth
    f = _page_figures()
    H, G = int(f["query_heads"]), int(f["kv_heads"])
    kB = int(f["selected_blocks"] * f["block_tokens"])
    assert kB == f["max_keys_per_query"]
    r = bench.paper_flop_ratio(H=H, G=G, d=128, dI=128, L=int(f["context_tokens"]), kB=kB)
    assert round(r, 1) == f["attention_flop_ratio_vs_gqa"]
    for name in ("prefill_L32768", "prefill_L131072", "prefill_L1048576_hot",
                 "decode_N64_L262144"):
        s = synth.WORKLOADS[name].shape
        assert (s.H, s.G, s.B, s.k) == (H, G, int(f["block_tokens"]), int(f["selected_blocks"]))
    assert synth.WORKLOADS["prefill_L1048576_hot"].shape.L == int(f["context_tokens"])


def test_paper_ratio_28_4():
    r = bench.paper_flop_ratio(H=64, G=4, d=128, dI=128, L=1 << 20, kB=2048)
    assert round(r, 1) == 28.4
    assert abs(r - 28.44) < 0.01
    # independent of d when dI = d
    assert abs(bench.paper_flop_ratio(64, 4, 64, 64, 1 << 20, 2048) - r) < 1e-9


def test_prefill_work_matches_closed_forms():
    L, H, G, d, dI, k = 131072, 64, 4, 128, 128, 16
    w = bench.prefill_work(L, H, G, d, dI, k)
    nb = L // 128
    # competitor keys: sum over query blocks b of 128 queries x 128*b keys
    assert w["pairs"] == 128 * 128 * nb * (nb - 1) / 2
    assert abs(w["flops"]["k1_index_pool"] - 8.79e12) / 8.79e12 < 1e-3
    # attended tokens per group: full budget minus the causal part of the own block
    assert abs(w["flops"]["k4_kv_outer"] - 8.46e12) / 8.46e12 < 2e-2
    dense = w["dense_gqa_flops"]
    assert abs(dense - 4 * H * d * L * (L + 1) / 2) < 1
    # at 1M the index branch dominates MSA's algorithmic FLOPs (~89%)
    w1 = bench.prefill_work(1 << 20, H, G, d, dI, k)
    frac = (w1["flops"]["k1_index_pool"] + w1["flops"]["k12_index_select"]) / w1["f_total"]
    assert 0.88 < frac < 0.90
    # the fused index kernel serves the query chunks whose rows are long: at 1M (chunks
    # of 131072 queries) chunks 1..7; at 128K (one chunk from query 0) none
    fused = bench.fused_index_rows(1 << 20, k)
    assert not fused[:131072].any() and fused[131072:].all()
    assert not bench.fused_index_rows(131072, k).any()
    assert not bench.fused_index_rows(1 << 20, 18).any()      # k - 1 > 16: K1 + K2 only
    # too few work-groups to fill the part: 16384-query chunks (256 at G = 4) stay on
    # K1 + K2, 65536-query chunks (1024) are fused
    assert not bench.fused_index_rows(131072, k, chunk=16384).any()
    f64 = bench.fused_index_rows(262144, k, chunk=65536)
    assert not f64[:65536].any() and f64[65536:].all()
    assert not bench.fused_index_rows(262144, k, chunk=65536, G=1).any()   # 512 at G = 1
    assert w["flops"]["k12_index_select"] == 0.0


def test_prefill_work_dense_sequences():
    """A sequence of at most k blocks keeps all its causal blocks in every row: its
    work is dense causal GQA attention (one kernel, no index branch)."""
    H, G, d, dI, k = 64, 4, 128, 128, 16
    for L in (512, 700, 2048):
        w = bench.prefill_work(L, H, G, d, dI, k)
        assert set(w["flops"]) == {"kd_dense"} and w["bytes"] == {}
        assert w["flops"]["kd_dense"] == 4 * H * d * L * (L + 1) / 2 == w["f_total"]
        assert w["pairs"] == 0.0
        # the sparse path attends exactly the same tokens
        assert w["attended_per_group"] == L * (L + 1) / 2
    w = bench.prefill_work(2049, H, G, d, dI, k)          # k + 1 blocks: the sparse path
    assert "kd_dense" not in w["flops"] and w["flops"]["k4_kv_outer"] > 0
    w = bench.prefill_work(512, H, G, d, dI, k, dense_main=False)   # given ids
    assert "kd_dense" not in w["flops"]
    assert bench.KERNEL_ROOF["kd_dense"] == "mfma"
    # staged K/V: a work-group holds 8 queries at r = 16; 64 tiles per 512 queries,
    # tile t stages blocks 0 .. 8t // 128
    staged = bench.prefill_work(512, H, G, d, dI, k)["design_bytes"]["kd_dense"]["kv_blocks_staged"]
    assert staged == 16 * (1 + 2 + 3 + 4) * G * 2 * 128 * d * 2


def test_decode_work():
    w = bench.decode_work(64, 262144, 64, 4, 128, 128, 16)
    # idx-K stream of all competitor blocks dominates: ~4 GiB of the ~4.57 GB step
    assert 4.2e9 < w["bytes"]["k1d_index_pool"] < 4.4e9
    assert 4.4e9 < w["total_bytes"] < 4.7e9


def test_kernel_roofs():
    """Each kernel is placed on the roof its work has: the index-score and the
    sparse-attention contractions on the bf16 matrix cores (2*G*dI FLOP per scored
    (query, key) pair, 4*r*d FLOP per attended (query, group, token)); selection,
    scheduling, combine and the decode stream on HBM bandwidth."""
    assert bench.KERNEL_ROOF["k1_index_pool"] == "mfma"
    assert bench.KERNEL_ROOF["k4_kv_outer"] == "mfma"
    for k in ("k2_select", "k3_schedule", "k5_combine", "k1d_index_pool", "k1d_index_pool_fp8",
              "k4d_merge", "k4d_split", "k4d_online", "k4d_parts"):
        assert bench.KERNEL_ROOF[k] == "hbm", k
    L, H, G, d, dI, k = 131072, 64, 4, 128, 128, 16
    w = bench.prefill_work(L, H, G, d, dI, k)
    # K4 at 13.2 ms per launch: its FLOPs over the bf16 peak, whatever bytes it moves
    r4 = bench.roofline("k4_kv_outer", w, 1, 13.2)
    assert r4["bound"] == "mfma" and r4["unit"] == "TFLOP/s"
    assert abs(r4["frac"] - w["flops"]["k4_kv_outer"] / 13.2e-3 / 2.5e15) < 1e-12
    assert 0.25 < r4["frac"] < 0.26
    # the gathered q rows and the partial round trip are the KV-outer design's bytes,
    # reported beside the FLOPs and never as the kernel's work
    assert set(r4["design_bytes_per_launch"]) == {"q_rows_gathered", "partial_rows_out",
                                                  "kv_blocks_staged"}
    assert "k4_kv_outer" not in w["bytes"] and "k1_index_pool" not in w["bytes"]
    r1 = bench.roofline("k1_index_pool", w, 1, 6.85)
    assert r1["bound"] == "mfma" and 0.50 < r1["frac"] < 0.52
    r5 = bench.roofline("k5_combine", w, 1, 6.28)
    assert r5["bound"] == "hbm" and r5["unit"] == "GB/s"
    wd = bench.decode_work(64, 262144, 64, 4, 128, 128, 16)
    rd = bench.roofline("k1d_index_pool", wd, 1, 0.7146)
    assert rd["bound"] == "hbm" and 0.74 < rd["frac"] < 0.76
