"""GPU parity: the HIP path (through the C ABI via the thin binding) against the
CPU oracle on the same seeded inputs.  Block ids bit-exact outside near-ties
(relative boundary gap < 1e-4); outputs within max-abs 2e-2 / mean-abs 2e-3."""
from __future__ import annotations

import math
import os
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _parity, _refs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[parity] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_idx_amd as msa  # noqa: F401  (fails loudly if not built)
    msa.load_library()
    yield
    torch.cuda.synchronize()


def _msa():
    import block_sparse_long_idx_amd as msa
    return msa


def _prefill_gpu(x, k, return_ids=True):
    msa = _msa()
    dev = {n: t.to(DEV) for n, t in x.items() if isinstance(t, torch.Tensor)}
    out, ids = msa.prefill(dev["q"], dev["k"], dev["v"], dev["iq"], dev["ik"], kslots=k,
                           return_ids=True)
    torch.cuda.synchronize()
    return out, ids


def _full_check(shape, seed, plant="lit", rows=None, **kw):
    _say(f"prefill L={shape.L} H={shape.H} G={shape.G} d={shape.d} dI={shape.dI} "
         f"k={shape.k} seed={seed} plant={plant}")
    x = synth.prefill_inputs(shape, seed=seed, plant=plant, **kw)
    out, ids = _prefill_gpu(x, shape.k)
    if rows is None:
        rows = np.arange(shape.L)
    scale = 1.0 / math.sqrt(shape.d)
    st = _parity.prefill_rows_vs_oracle(x, rows, ids.cpu().numpy()[rows],
                                        out.float().cpu().numpy()[rows], 128, shape.k, scale)
    _say(f"  -> {st}")
    assert st["id_mismatches"] == 0
    assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS
    return st, out, ids


TINY = synth.WORKLOADS["tiny_prefill_L4096"].shape


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("plant", ["lit", "hot"])
def test_tiny_prefill_full(seed, plant):
    _full_check(TINY, seed, plant)


def test_select_blocks_tiny():
    msa = _msa()
    x = synth.prefill_inputs(TINY, seed=3)
    _say("select_blocks tiny")
    ids = msa.select_blocks(x["iq"].to(DEV), x["ik"].to(DEV), k=TINY.k).cpu().numpy()
    S = oracle.block_scores(x["iq"], x["ik"], 128)
    rows = np.arange(TINY.L)
    oids, gap = oracle.select(S, rows, 128, TINY.k)
    _parity.check_selection_valid(ids, rows, TINY.k)
    tie, nmis = _parity.compare_ids(ids, oids, gap)
    assert nmis == 0
    tr = np.nonzero(tie.any(axis=1))[0]
    _parity.check_near_tie_band(ids[tr], oids[tr], S[tr], rows[tr])


def test_sparse_attn_with_oracle_ids():
    """Main branch alone, fed the oracle's ids (decoupled from selection)."""
    msa = _msa()
    x = synth.prefill_inputs(TINY, seed=4)
    scale = 1.0 / math.sqrt(TINY.d)
    ids, gap, ref = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], 128, TINY.k, scale)
    _say("sparse_attn with oracle ids")
    out = msa.sparse_attn(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                          torch.from_numpy(ids).to(DEV)).float().cpu().numpy()
    mx, mean = _parity.compare_out(out, ref)
    _say(f"  -> max {mx:.3e} mean {mean:.3e}")
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS
    # arbitrary valid ids (not from the index branch), including -1 padding
    rng = np.random.default_rng(0)
    ids2 = np.full_like(ids, -1)
    for i in range(TINY.L):
        bi = i // 128
        for g in range(TINY.G):
            m = int(rng.integers(0, min(TINY.k - 1, bi) + 1))
            ch = sorted(list(rng.choice(bi, size=m, replace=False)) + [bi]) if bi else [0]
            ids2[i, g, :len(ch)] = ch
    ref2 = oracle.attend(x["q"], x["k"], x["v"], ids2, 128, scale)
    out2 = msa.sparse_attn(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV),
                           torch.from_numpy(ids2).to(DEV)).float().cpu().numpy()
    mx, mean = _parity.compare_out(out2, ref2)
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS


def _sparse_attn_skewed_check(shape, hot, seed, rows):
    msa = _msa()
    _say(f"sparse_attn skewed ids L={shape.L} H={shape.H} G={shape.G} hot={hot} seed={seed}")
    x = synth.prefill_inputs(shape, seed=seed, plant="none", device=DEV)
    ids = synth.skewed_ids(shape.L, shape.G, shape.k, hot=hot, seed=seed, device=DEV)
    out = msa.sparse_attn(x["q"], x["k"], x["v"], ids)
    torch.cuda.synchronize()
    rows_t = torch.from_numpy(rows).to(DEV)
    _say(f"  oracle on {len(rows)} rows")
    # the oracle takes the ids of the listed rows only
    ref = oracle.attend(x["q"].cpu(), x["k"].cpu(), x["v"].cpu(), ids[rows_t].cpu().numpy(), 128,
                        1.0 / math.sqrt(shape.d), rows=rows)
    mx, mean = _parity.compare_out(out[rows_t].float().cpu().numpy(), ref)
    _say(f"  -> max {mx:.3e} mean {mean:.3e}")
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS
    return ids


def test_sparse_attn_skewed_ids_8k():
    """Main branch alone on constructed ids with blocks 0-3 in every row (their lists
    split into many tiles), rows of every block checked."""
    shape = synth.PrefillShape(L=8192, H=64, G=4, d=128, dI=128, B=128, k=16)
    _sparse_attn_skewed_check(shape, (0, 1, 2, 3), 3, _sample_rows(shape.L, 1024, 3))


def test_sparse_attn_skewed_ids_128k_bench_config():
    """The benchmark's constructed-skew workload (L = 131072, one query chunk, blocks
    0-3 hot: 1024 tiles per hot list and group) on sampled rows."""
    wl = synth.WORKLOADS["sparse_attn_L131072_skewed"]
    ids = _sparse_attn_skewed_check(wl.shape, wl.hot_blocks, 0, _sample_rows(wl.shape.L, 768, 4))
    assert (ids[128 * 16:, :, :4].cpu() == torch.arange(4, dtype=torch.int32)).all()


@pytest.mark.parametrize("L", [1, 127, 128, 129, 1000, 4097])
def test_ragged_lengths(L):
    shape = synth.PrefillShape(L=L, H=8, G=2, d=64, dI=32, B=128, k=4)
    _full_check(shape, seed=5)


@pytest.mark.parametrize("H,G,d,dI,k", [
    (64, 4, 128, 128, 16),   # the pages' research-model shape
    (16, 8, 64, 64, 3),
    (32, 1, 128, 128, 5),    # 32 query heads per group
    (4, 4, 64, 32, 1),       # one head per group; local block only
    (8, 2, 128, 64, 32),     # k = 32 slots
])
def test_shape_grid(H, G, d, dI, k):
    shape = synth.PrefillShape(L=2000, H=H, G=G, d=d, dI=dI, B=128, k=k)
    _full_check(shape, seed=6)


@pytest.mark.parametrize("H,G,d,dI,k", [
    (16, 8, 64, 64, 6),      # eight groups (32 queries per K1 work-group)
    (32, 1, 128, 128, 5),    # one group
    (8, 2, 64, 32, 7),       # index dim 32
])
def test_shape_grid_long(H, G, d, dI, k):
    """Long enough (97 blocks, four key chunks of K1) that every group really
    selects k-1 of many competitors."""
    shape = synth.PrefillShape(L=12345, H=H, G=G, d=d, dI=dI, B=128, k=k)
    _full_check(shape, seed=16, rows=_sample_rows(shape.L, 1200, 16))


def test_determinism():
    x = synth.prefill_inputs(TINY, seed=7)
    _say("determinism")
    o1, i1 = _prefill_gpu(x, TINY.k)
    o2, i2 = _prefill_gpu(x, TINY.k)
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def _sample_rows(L, n, seed):
    rng = np.random.default_rng(seed)
    head = np.arange(min(L, 256))
    tail = np.arange(max(0, L - 128), L)
    mid = rng.choice(L, size=min(n, L), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_32k_sampled(seed):
    """The 32K workload: the first two blocks, the last block and 2048 uniform rows
    (512 for seeds other than 0)."""
    shape = synth.WORKLOADS["prefill_L32768"].shape
    _full_check(shape, seed=seed, rows=_sample_rows(shape.L, 2048 if seed == 0 else 512, seed))


def test_hot_blocks_16k_sampled():
    """Blocks 0-3 picked by (nearly) every query: long lists split over many tiles."""
    shape = synth.PrefillShape(L=16384, H=64, G=4, d=128, dI=128, B=128, k=16)
    st, out, ids = _full_check(shape, seed=1, plant="hot", rows=_sample_rows(shape.L, 512, 1),
                               n_plant=0, c=3.0, hot_blocks=(0, 1, 2, 3))
    idn = ids.cpu().numpy()
    late = idn[1024:]
    frac = np.mean([(late[:, :, :4] == np.arange(4)).all(-1).mean()])
    _say(f"  hot-block selection fraction {frac:.4f}")
    assert frac > 0.99


def test_prefill_ragged_100003_sampled():
    """A long sequence whose last block is partial (100003 = 781 * 128 + 35 tokens):
    the first two blocks, the last block and 1024 uniform rows."""
    shape = synth.PrefillShape(L=100003, H=64, G=4, d=128, dI=128, B=128, k=16)
    _full_check(shape, seed=11, rows=_sample_rows(shape.L, 1024, 11))


def test_determinism_128k():
    """The 128K workload twice: ids and outputs bitwise equal, although the order of
    entries inside the scheduler's lists follows LDS atomic timing."""
    wl = synth.WORKLOADS["prefill_L131072"]
    s = wl.shape
    _say("determinism 128K")
    x = synth.prefill_inputs(s, seed=5, plant=wl.plant, device=DEV)
    msa = _msa()
    runs = []
    for _ in range(2):
        out, ids = msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=s.k,
                               return_ids=True)
        torch.cuda.synchronize()
        runs.append((out, ids))
    assert torch.equal(runs[0][1], runs[1][1])
    assert torch.equal(runs[0][0].view(torch.int16), runs[1][0].view(torch.int16))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_prefill_128k_sampled(seed):
    """The 128K workload in the launch configuration the benchmark times (2048 uniform
    rows for seed 0, 512 for the others, plus the first two and the last block)."""
    wl = synth.WORKLOADS["prefill_L131072"]
    shape = wl.shape
    _say(f"prefill 128K seed {seed}: generate on GPU")
    x = synth.prefill_inputs(shape, seed=seed, plant=wl.plant, device=DEV)
    msa = _msa()
    out, ids = msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=shape.k,
                           return_ids=True)
    torch.cuda.synchronize()
    # the first two blocks, the last block and uniform rows
    rows = _sample_rows(shape.L, 2048 if seed == 0 else 512, 2 + seed)
    _say(f"  oracle on {len(rows)} rows")
    st = _parity.prefill_rows_vs_oracle(x, rows, ids[rows].cpu().numpy(),
                                        out[rows].float().cpu().numpy(), 128, shape.k,
                                        1.0 / math.sqrt(shape.d))
    _say(f"  -> {st}")
    assert st["id_mismatches"] == 0
    assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS
    # every row's selection is valid
    _parity.check_selection_valid(ids.cpu().numpy(), np.arange(shape.L), shape.k)


@pytest.mark.parametrize("H,G,d,dI,k", [
    (32, 8, 64, 64, 8),       # eight index groups, d = 64, four heads per group
    (64, 2, 128, 64, 32),     # 32 heads per group, index dim 64, k = 32 slots
])
def test_shape_grid_64k_sampled(H, G, d, dI, k):
    """Other head groupings at a length where every K1 work-group scores full key
    chunks and K4 runs many tiles per list; inputs drawn on the GPU, oracle on
    sampled rows."""
    shape = synth.PrefillShape(L=65536, H=H, G=G, d=d, dI=dI, B=128, k=k)
    _say(f"prefill L={shape.L} H={H} G={G} d={d} dI={dI} k={k}: generate on GPU")
    x = synth.prefill_inputs(shape, seed=21, device=DEV)
    out, ids = _msa().prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=k,
                              return_ids=True)
    torch.cuda.synchronize()
    rows = _sample_rows(shape.L, 160, 21)
    st = _parity.prefill_rows_vs_oracle(x, rows, ids[rows].cpu().numpy(),
                                        out[rows].float().cpu().numpy(), 128, k,
                                        1.0 / math.sqrt(d))
    _say(f"  -> {st}")
    assert st["id_mismatches"] == 0
    assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS
    _parity.check_selection_valid(ids.cpu().numpy(), np.arange(shape.L), k)


# ------------------------------- decode ------------------------------------
def _decode_check(shape, seq_len, seed, seqs=None, device="cpu"):
    msa = _msa()
    _say(f"decode N={shape.N} Lmax={shape.Lc} seq_len[:8]={list(seq_len[:8])} seed={seed}")
    x = synth.decode_inputs(shape, seed=seed, seq_len=np.clip(seq_len, 1, shape.Lc), device=device)
    sl = torch.tensor(np.asarray(seq_len, np.int32), device=DEV)
    d = {n: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for n, t in x.items()}
    out, ids = msa.decode(d["q"], d["iq"], d["k_cache"], d["v_cache"], d["ik_cache"], sl,
                          kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    out = out.float().cpu().numpy()
    ids = ids.cpu().numpy()
    valid = (np.asarray(seq_len) >= 1) & (np.asarray(seq_len) <= shape.Lc)
    if seqs is None:
        seqs = np.nonzero(valid)[0]
    scale = 1.0 / math.sqrt(shape.d)
    oids, gap, oout = oracle.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"],
                                    np.clip(seq_len, 1, shape.Lc), 128, shape.k, scale, seqs=seqs)
    pos = np.asarray(seq_len)[seqs] - 1
    _parity.check_selection_valid(ids[seqs], pos, shape.k)
    tie, nmis = _parity.compare_ids(ids[seqs], oids, gap)
    ref = oout.copy()
    banded = 0
    if tie.any():
        tr = np.nonzero(tie.any(axis=1))[0]
        lens_t = np.clip(seq_len, 1, shape.Lc)[seqs[tr]]
        sel = torch.as_tensor(seqs[tr], device=x["iq"].device)
        S = oracle.decode_block_scores(x["iq"][sel], x["ik_cache"][sel], lens_t, 128,
                                       np.arange(len(tr)))
        banded = _parity.check_near_tie_band(ids[seqs[tr]], oids[tr], S, lens_t - 1)
        ref[tr] = oracle.decode_attend(x["q"], x["k_cache"], x["v_cache"],
                                       np.clip(seq_len, 1, shape.Lc), ids[seqs[tr]], 128, scale,
                                       seqs[tr])
    mx, mean = _parity.compare_out(out[seqs], ref)
    _say(f"  -> near_ties {int(tie.sum())} (band checked {banded}) mismatches {nmis} "
         f"max {mx:.3e} mean {mean:.3e}")
    assert nmis == 0
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS
    for n in np.nonzero(~valid)[0]:
        assert (ids[n] == -1).all() and (out[n] == 0).all()


def test_decode_small_ragged():
    shape = synth.DecodeShape(N=8, Lc=2000, H=64, G=4, d=128, dI=128, B=128, k=16)
    seq_len = np.array([1, 127, 128, 129, 2000, 1500, 0, 2001])   # last two invalid
    _decode_check(shape, seq_len, seed=0)


def test_decode_tiny_dims():
    shape = synth.DecodeShape(N=5, Lc=4096, H=8, G=2, d=64, dI=32, B=128, k=4)
    _decode_check(shape, np.array([4096, 3000, 129, 640, 1]), seed=1)


@pytest.mark.parametrize("N,G,k", [(128, 4, 16), (160, 4, 32), (9, 2, 1)])
def test_decode_one_launch_attention(N, G, k):
    """Decode attention in one launch (one work-group per (sequence, group), running
    merge in registers): the form used once a launch has at least 512 (sequence,
    group) pairs, or with k = 1; smaller batches split each pair's slots into parts
    merged by the combine.  Ragged lengths, some past the cache, some of one token."""
    shape = synth.DecodeShape(N=N, Lc=3000, H=4 * G, G=G, d=128, dI=128, B=128, k=k)
    rng = np.random.default_rng(N)
    seq_len = rng.integers(1, shape.Lc + 1, N)
    seq_len[:4] = [1, 129, shape.Lc, shape.Lc + 7][:min(4, N)]
    _decode_check(shape, seq_len, seed=N)


@pytest.mark.parametrize("H,G,d,dI,k", [(64, 8, 64, 64, 8), (16, 1, 128, 128, 16),
                                         (32, 1, 128, 128, 4), (64, 2, 128, 128, 16),
                                         (32, 1, 64, 32, 8)])
def test_decode_other_groupings(H, G, d, dI, k):
    """Other head groupings; 32 heads per group run the 32-column decode forms (slots
    merged in LDS where they fit: k = 4 at d = 128, k = 8 at d = 64; else the split
    form and the combine: k = 16 at d = 128)."""
    shape = synth.DecodeShape(N=6, Lc=20000, H=H, G=G, d=d, dI=dI, B=128, k=k)
    _decode_check(shape, np.array([20000, 17000, 129, 2048, 1, 9999]), seed=12)


def test_decode_k32_ragged():
    """k = 32 slots (4096 keys per query) over ragged lengths."""
    shape = synth.DecodeShape(N=6, Lc=30000, H=64, G=4, d=128, dI=128, B=128, k=32)
    _decode_check(shape, np.array([30000, 4095, 4096, 4097, 129, 22222]), seed=13)


def test_decode_full_size_ragged_lengths():
    """The full-size cache (64 x 262144) with random lengths from 1 to 262144: short
    sequences, partial own blocks, and the oracle on every sequence."""
    shape = synth.WORKLOADS["decode_N64_L262144"].shape
    rng = np.random.default_rng(21)
    seq_len = rng.integers(1, shape.Lc + 1, shape.N)
    seq_len[:4] = [1, 128, 129, shape.Lc]
    _decode_check(shape, seq_len, seed=21, device=DEV)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_decode_full_size_all_sequences(seed):
    """64 sequences x 262144 cached tokens (the one-launch attention with its running
    merge); oracle on every sequence, three seeds."""
    wl = synth.WORKLOADS["decode_N64_L262144"]
    shape = wl.shape
    seq_len = np.full(shape.N, shape.Lc)
    _decode_check(shape, seq_len, seed=seed, device=DEV)


# ------------------------- varlen / prefix prefill ---------------------------
def _cat_inputs(parts):
    return {n: torch.cat([p[n] for p in parts]) for n in ("q", "k", "v", "iq", "ik")}


def test_prefill_varlen_batch():
    """Five packed sequences without prefix: each equals its own msa_prefill bitwise
    and matches the oracle on every row."""
    msa = _msa()
    lens = [1000, 128, 1, 4097, 3000]
    shapes = [synth.PrefillShape(L=L, H=16, G=4, d=128, dI=128, B=128, k=8) for L in lens]
    xs = [synth.prefill_inputs(sh, seed=30 + i) for i, sh in enumerate(shapes)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    _say(f"varlen prefill lens={lens}")
    c = {n: t.to(DEV) for n, t in _cat_inputs(xs).items()}
    out, ids = msa.prefill_varlen(c["q"], c["k"], c["v"], c["iq"], c["ik"], cu, cu, kslots=8,
                                  return_ids=True)
    torch.cuda.synchronize()
    for i, (sh, x) in enumerate(zip(shapes, xs)):
        sl = slice(int(cu[i]), int(cu[i + 1]))
        o1, i1 = _prefill_gpu(x, sh.k)
        assert torch.equal(ids[sl], i1)
        assert torch.equal(out[sl].view(torch.int16), o1.view(torch.int16))
        st = _parity.prefill_rows_vs_oracle(x, np.arange(sh.L), i1.cpu().numpy(),
                                            o1.float().cpu().numpy(), 128, sh.k,
                                            1.0 / math.sqrt(sh.d))
        _say(f"  seq {i} L={sh.L} -> {st}")
        assert st["id_mismatches"] == 0
        assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS


def test_prefill_with_cached_prefix():
    """Chunked prefill over cached prefixes (first P tokens' K/V/idx-K already in the
    cache, only the last L - P tokens are queries): rows P.. of the whole-sequence
    prefill, bitwise, and the oracle on those rows."""
    msa = _msa()
    lens, prefixes = [5000, 2048, 700, 1300], [1024, 1920, 0, 1280]
    shapes = [synth.PrefillShape(L=L, H=16, G=4, d=128, dI=128, B=128, k=8) for L in lens]
    xs = [synth.prefill_inputs(sh, seed=40 + i) for i, sh in enumerate(shapes)]
    _say(f"prefix prefill lens={lens} prefixes={prefixes}")
    new = [{"q": x["q"][P:], "iq": x["iq"][P:]} for x, P in zip(xs, prefixes)]
    cu_q = np.concatenate([[0], np.cumsum([L - P for L, P in zip(lens, prefixes)])])
    cu_kv = np.concatenate([[0], np.cumsum(lens)])
    q = torch.cat([n_["q"] for n_ in new]).to(DEV)
    iq = torch.cat([n_["iq"] for n_ in new]).to(DEV)
    kk = torch.cat([x["k"] for x in xs]).to(DEV)
    vv = torch.cat([x["v"] for x in xs]).to(DEV)
    ik = torch.cat([x["ik"] for x in xs]).to(DEV)
    out, ids = msa.prefill_varlen(q, kk, vv, iq, ik, cu_q, cu_kv, kslots=8, return_ids=True)
    torch.cuda.synchronize()
    for i, (sh, x, P) in enumerate(zip(shapes, xs, prefixes)):
        sl = slice(int(cu_q[i]), int(cu_q[i + 1]))
        o1, i1 = _prefill_gpu(x, sh.k)
        assert torch.equal(ids[sl], i1[P:])
        assert torch.equal(out[sl].view(torch.int16), o1[P:].view(torch.int16))
        rows = np.arange(P, sh.L)
        st = _parity.prefill_rows_vs_oracle(x, rows, ids[sl].cpu().numpy(),
                                            out[sl].float().cpu().numpy(), 128, sh.k,
                                            1.0 / math.sqrt(sh.d))
        _say(f"  seq {i} L={sh.L} P={P} -> {st}")
        assert st["id_mismatches"] == 0
        assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS


def _packed_case(lens, prefixes, shape_kw, seed):
    """Packed varlen inputs: new tokens of every sequence (q, idx_q) and all tokens
    (k, v, idx_k), plus the per-sequence whole inputs."""
    shapes = [synth.PrefillShape(L=L, B=128, **shape_kw) for L in lens]
    xs = [synth.prefill_inputs(sh, seed=seed + i) for i, sh in enumerate(shapes)]
    cu_q = np.concatenate([[0], np.cumsum([L - P for L, P in zip(lens, prefixes)])])
    cu_kv = np.concatenate([[0], np.cumsum(lens)])
    packed = {
        "q": torch.cat([x["q"][P:] for x, P in zip(xs, prefixes)]).to(DEV),
        "iq": torch.cat([x["iq"][P:] for x, P in zip(xs, prefixes)]).to(DEV),
        "k": torch.cat([x["k"] for x in xs]).to(DEV),
        "v": torch.cat([x["v"] for x in xs]).to(DEV),
        "ik": torch.cat([x["ik"] for x in xs]).to(DEV),
    }
    return shapes, xs, cu_q, cu_kv, packed


def _varlen(c, cu_q, cu_kv, k, workspace=None):
    msa = _msa()
    out, ids = msa.prefill_varlen(c["q"], c["k"], c["v"], c["iq"], c["ik"], cu_q, cu_kv, kslots=k,
                                  return_ids=True, workspace=workspace)
    torch.cuda.synchronize()
    return out, ids


def _short_batch(n, seed, max_len=700):
    """n sequence lengths in [1, max_len] (boundary lengths first) and prefixes: every
    third sequence longer than 128 tokens continues a cached prefix of whole blocks."""
    rng = np.random.default_rng(seed)
    lens = [1, 127, 128, 129, 255, 256, 257, 640] + list(rng.integers(1, max_len + 1, n - 8))
    prefixes = [(int(rng.integers(1, L // 128 + 1)) * 128 if (i % 3 == 0 and L > 128) else 0)
                for i, L in enumerate(lens)]
    prefixes = [P if P < L else P - 128 for P, L in zip(prefixes, lens)]
    return [int(L) for L in lens], prefixes


def test_prefill_varlen_many_short_sequences():
    """150 sequences of 1 to 700 tokens, a third of them continuing a cached prefix,
    at k = 4: those of at most 512 tokens go to the dense kernel (one launch), the
    others run in batches of one launch set each (ended by the dense ones between
    them).  Every sequence's rows equal its own whole-sequence prefill bitwise;
    sampled rows match the oracle."""
    kw = dict(H=16, G=4, d=128, dI=128, k=4)
    lens, prefixes = _short_batch(150, seed=61)
    _say(f"varlen 150 short sequences, {sum(lens)} tokens, {sum(L - P for L, P in zip(lens, prefixes))} new")
    shapes, xs, cu_q, cu_kv, c = _packed_case(lens, prefixes, kw, seed=600)
    out, ids = _varlen(c, cu_q, cu_kv, kw["k"])
    checked = 0
    for i, (sh, x, P) in enumerate(zip(shapes, xs, prefixes)):
        sl = slice(int(cu_q[i]), int(cu_q[i + 1]))
        o1, i1 = _prefill_gpu(x, sh.k)
        assert torch.equal(ids[sl], i1[P:]), f"sequence {i} (L={sh.L}, P={P}): ids"
        assert torch.equal(out[sl].view(torch.int16), o1[P:].view(torch.int16)), \
            f"sequence {i} (L={sh.L}, P={P}): out"
        if i % 10 == 0:
            rows = np.unique(np.array([P, (P + sh.L) // 2, sh.L - 1]))
            st = _parity.prefill_rows_vs_oracle(x, rows, i1.cpu().numpy()[rows],
                                                o1.float().cpu().numpy()[rows], 128, sh.k,
                                                1.0 / math.sqrt(sh.d))
            assert st["id_mismatches"] == 0
            assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS
            checked += len(rows)
    _say(f"  150 sequences bitwise equal to their own prefill; {checked} rows vs the oracle")


def test_prefill_varlen_batching_is_invisible():
    """The same packed batch with three workspaces -- the full size (every batch
    formed), a third of it (smaller batches) and the minimum (every sequence alone)
    -- gives bitwise the same outputs and ids; also for d = 64, dI = 32, G = 2."""
    msa = _msa()
    for kw, seed in ((dict(H=16, G=4, d=128, dI=128, k=8), 700),
                     (dict(H=8, G=2, d=64, dI=32, k=4), 800)):
        lens, prefixes = _short_batch(40, seed=seed, max_len=1500)
        shapes, xs, cu_q, cu_kv, c = _packed_case(lens, prefixes, kw, seed=seed)
        full = msa.workspace_size("prefill_varlen", cu_q=cu_q, cu_kv=cu_kv, **kw)
        single = msa.workspace_size("prefill", L=max(lens), **kw)
        o_ref, i_ref = _varlen(c, cu_q, cu_kv, kw["k"])
        for nbytes in (full // 3, min(single, full // 8)):
            _say(f"varlen {kw} workspace {nbytes} of {full}")
            o, i = _varlen(c, cu_q, cu_kv, kw["k"], workspace=msa._workspace(nbytes, DEV))
            assert torch.equal(i, i_ref)
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        # and the first sequences against their own prefill
        for j in range(4):
            sl = slice(int(cu_q[j]), int(cu_q[j + 1]))
            o1, i1 = _prefill_gpu(xs[j], shapes[j].k)
            assert torch.equal(o_ref[sl].view(torch.int16), o1[prefixes[j]:].view(torch.int16))


def test_prefill_varlen_long_and_short_mixed():
    """Short sequences around one with more than 8192 new tokens: batches {1300, 1500},
    the long one alone, then {1100, 1200}, and the one-token sequence (at most k
    blocks) on the dense kernel.  Every sequence's rows equal its own whole-sequence
    prefill bitwise."""
    kw = dict(H=16, G=4, d=128, dI=128, k=8)
    lens, prefixes = [1300, 1500, 9000, 1100, 1200, 1], [0, 384, 256, 0, 128, 0]
    shapes, xs, cu_q, cu_kv, c = _packed_case(lens, prefixes, kw, seed=900)
    _say(f"varlen mixed lens={lens} prefixes={prefixes}")
    out, ids = _varlen(c, cu_q, cu_kv, kw["k"])
    for i, (sh, x, P) in enumerate(zip(shapes, xs, prefixes)):
        sl = slice(int(cu_q[i]), int(cu_q[i + 1]))
        o1, i1 = _prefill_gpu(x, sh.k)
        assert torch.equal(ids[sl], i1[P:]), f"sequence {i}: ids"
        assert torch.equal(out[sl].view(torch.int16), o1[P:].view(torch.int16)), f"sequence {i}"


def test_prefill_varlen_256x512_bench_config():
    """The benchmark's packed-prompt workload in its launch configuration: 256 prompts
    of 512 tokens (H = 64, G = 4, d = dI = 128, k = 16), at most k blocks each, so two
    dense-kernel launches of 128, the workspace sized by
    msa_prefill_varlen_workspace_size.  Sampled prompts equal
    their own prefill bitwise; sampled rows match the oracle."""
    msa = _msa()
    wl = synth.WORKLOADS["prefill_varlen_256x512"]
    s = wl.shape
    _say("varlen 256 x 512 (benchmark configuration)")
    parts = [synth.prefill_inputs(s, seed=b, plant=wl.plant, n_plant=wl.n_plant, c=wl.c,
                                  device=DEV) for b in range(wl.batch)]
    c = {n: torch.cat([p_[n] for p_ in parts]) for n in ("q", "k", "v", "iq", "ik")}
    cu = [b * s.L for b in range(wl.batch + 1)]
    ws = msa._workspace(msa.workspace_size("prefill_varlen", cu_q=cu, cu_kv=cu, H=s.H, G=s.G,
                                           d=s.d, dI=s.dI, k=s.k), DEV)
    out, ids = _varlen(c, cu, cu, s.k, workspace=ws)
    for b in (0, 1, 127, 128, 200, 255):
        sl = slice(cu[b], cu[b + 1])
        o1, i1 = msa.prefill(parts[b]["q"], parts[b]["k"], parts[b]["v"], parts[b]["iq"],
                             parts[b]["ik"], kslots=s.k, return_ids=True)
        torch.cuda.synchronize()
        assert torch.equal(ids[sl], i1) and torch.equal(out[sl].view(torch.int16),
                                                        o1.view(torch.int16)), f"prompt {b}"
        if b in (0, 200):
            host = {n: parts[b][n].cpu() for n in ("q", "k", "v", "iq", "ik")}
            rows = np.array([0, 127, 128, 300, 511])
            st = _parity.prefill_rows_vs_oracle(host, rows, i1.cpu().numpy()[rows],
                                                o1.float().cpu().numpy()[rows], 128, s.k,
                                                1.0 / math.sqrt(s.d))
            _say(f"  prompt {b} -> {st}")
            assert st["id_mismatches"] == 0
            assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS


@pytest.mark.parametrize("H,G,d,k,L", [
    (64, 4, 128, 16, 2048),   # exactly k blocks, 16 heads per group
    (8, 8, 64, 4, 385),       # one head per group; last block of one token
    (16, 8, 128, 8, 1000),    # 2 heads per group
    (32, 8, 64, 2, 256),      # 4 heads per group, two whole blocks
    (64, 8, 128, 3, 300),     # 8 heads per group
    (32, 1, 128, 2, 129),     # 32 heads per group
    (16, 4, 64, 1, 77),       # k = 1, one partial block
    (8, 2, 64, 6, 1),         # one token
])
def test_dense_sequences(H, G, d, k, L):
    """Sequences of at most k blocks (every row keeps all its causal blocks): the
    dense kernel against the oracle on every row, for each head-per-group width and
    both head dims; and against the general path (msa_select_blocks, then
    msa_sparse_attn on its ids): the same ids, outputs within rounding."""
    msa = _msa()
    shape = synth.PrefillShape(L=L, H=H, G=G, d=d, dI=64, B=128, k=k)
    st, out, ids = _full_check(shape, seed=L + H)
    x = synth.prefill_inputs(shape, seed=L + H)
    dev = {n: t_.to(DEV) for n, t_ in x.items() if isinstance(t_, torch.Tensor)}
    ids2 = msa.select_blocks(dev["iq"], dev["ik"], k=k)
    out2 = msa.sparse_attn(dev["q"], dev["k"], dev["v"], ids2)
    torch.cuda.synchronize()
    assert torch.equal(ids, ids2)
    diff = (out.float() - out2.float()).abs()
    _say(f"  vs general path: max {diff.max().item():.3g}")
    assert diff.max().item() < _parity.MAX_ABS


def test_dense_sequences_packed_launches():
    """150 dense sequences (k = 16, 1 to 2048 tokens, a third continuing a cached
    prefix) in one msa_prefill_varlen call: two dense launches (128 + 22 members),
    every sequence's rows bitwise equal to its own whole-sequence prefill."""
    kw = dict(H=16, G=4, d=128, dI=64, k=16)
    lens, prefixes = _short_batch(150, seed=71, max_len=2048)
    shapes, xs, cu_q, cu_kv, c = _packed_case(lens, prefixes, kw, seed=1700)
    _say(f"dense packed: {len(lens)} sequences, {sum(lens)} tokens")
    out, ids = _varlen(c, cu_q, cu_kv, kw["k"])
    for i, (sh, x, P) in enumerate(zip(shapes, xs, prefixes)):
        sl = slice(int(cu_q[i]), int(cu_q[i + 1]))
        o1, i1 = _prefill_gpu(x, sh.k)
        assert torch.equal(ids[sl], i1[P:]), f"sequence {i} (L={sh.L}, P={P}): ids"
        assert torch.equal(out[sl].view(torch.int16), o1[P:].view(torch.int16)), \
            f"sequence {i} (L={sh.L}, P={P}): out"


def test_prefix_prefill_32k_matches_whole():
    """L = 32768 with the first 16384 tokens cached: bitwise the second half of the
    whole-sequence prefill (a property that holds at any size)."""
    msa = _msa()
    wl = synth.WORKLOADS["prefill_L32768"]
    sh = wl.shape
    P = 16384
    x = synth.prefill_inputs(sh, seed=1, device=DEV)
    _say(f"prefix prefill L={sh.L} P={P}")
    o1, i1 = msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=sh.k, return_ids=True)
    out, ids = msa.prefill_varlen(x["q"][P:].contiguous(), x["k"], x["v"],
                                  x["iq"][P:].contiguous(), x["ik"], [0, sh.L - P], [0, sh.L],
                                  kslots=sh.k, return_ids=True)
    torch.cuda.synchronize()
    assert torch.equal(ids, i1[P:])
    assert torch.equal(out.view(torch.int16), o1[P:].view(torch.int16))


_BF16_NAN = 0x7FC0


def _poison_past_len(cache: torch.Tensor, seq_len) -> torch.Tensor:
    """A copy of a per-sequence cache [N, Lmax, ...] whose rows at and past each
    sequence's length hold bf16 NaN (rows a decode may not read)."""
    c = cache.clone()
    v = c.view(torch.int16)
    for n, L in enumerate(seq_len):
        v[n, int(L):] = _BF16_NAN
    return c


@pytest.mark.parametrize("N,k,Lc", [(6, 8, 2000), (6, 32, 5000), (64, 16, 1500)])
def test_decode_ignores_rows_past_seq_len(N, k, Lc):
    """Cache rows at and past seq_len are not part of the sequence (not yet written):
    NaN there must change neither the ids nor a single output bit.  Six sequences run
    the attention in parts merged by the combine; 64 sequences x 4 groups run it in
    one launch with the running merge."""
    msa = _msa()
    shape = synth.DecodeShape(N=N, Lc=Lc, H=16, G=4, d=128, dI=128, B=128, k=k)
    seq_len = np.array([1, 130, Lc // 2 + 5, Lc - 1, Lc, 700])
    if N > 6:
        seq_len = np.concatenate([seq_len, np.random.default_rng(N).integers(1, Lc + 1, N - 6)])
    _say(f"decode NaN past seq_len N={N} k={k} Lc={Lc} seq_len[:8]={list(seq_len[:8])}")
    x = synth.decode_inputs(shape, seed=12, seq_len=seq_len)
    sl = torch.tensor(seq_len.astype(np.int32), device=DEV)
    d = {n: x[n].to(DEV) for n in ("q", "iq", "k_cache", "v_cache", "ik_cache")}
    o1, i1 = msa.decode(d["q"], d["iq"], d["k_cache"], d["v_cache"], d["ik_cache"], sl,
                        kslots=k, return_ids=True)
    bad = {n: _poison_past_len(d[n], seq_len) for n in ("k_cache", "v_cache", "ik_cache")}
    o2, i2 = msa.decode(d["q"], d["iq"], bad["k_cache"], bad["v_cache"], bad["ik_cache"], sl,
                        kslots=k, return_ids=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert not torch.isnan(o2.float()).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_paged_decode_ignores_rows_past_seq_len():
    """Paged decode: the rows of a sequence's last page past its length hold NaN
    (a page being filled); ids and outputs must be bitwise those of clean pages."""
    msa = _msa()
    shape = synth.DecodeShape(N=5, Lc=2000, H=16, G=4, d=128, dI=128, B=128, k=16)
    seq_len = np.array([1, 129, 1000, 1999, 640])
    _say(f"paged decode NaN past seq_len seq_len={list(seq_len)}")
    x = synth.decode_inputs(shape, seed=13, seq_len=seq_len)
    pg = synth.paginate({n: x[n] for n in ("k_cache", "v_cache", "ik_cache")}, 128, 13,
                        extra_pages=2)
    g = {n: t.to(DEV) for n, t in pg.items()}
    q, iq = x["q"].to(DEV), x["iq"].to(DEV)
    sl = torch.tensor(seq_len.astype(np.int32), device=DEV)
    o1, i1 = msa.decode_paged(q, iq, g["k_pages"], g["v_pages"], g["ik_pages"], g["block_table"],
                              sl, kslots=shape.k, return_ids=True)
    bad = {n: g[n].clone() for n in ("k_pages", "v_pages", "ik_pages")}
    for n, L in enumerate(seq_len):
        b = (int(L) - 1) // 128
        page = int(pg["block_table"][n, b])
        for name in bad:
            bad[name].view(torch.int16)[page, int(L) - 128 * b:] = _BF16_NAN
    o2, i2 = msa.decode_paged(q, iq, bad["k_pages"], bad["v_pages"], bad["ik_pages"],
                              g["block_table"], sl, kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert not torch.isnan(o2.float()).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ----------------------------- paged decode ---------------------------------
def _compact_pages(pg, table, seqs, seq_len, B=128):
    """CPU copies of only the pages the listed sequences need, with their table
    rows renumbered; entries outside [0, num_pages) stay out of range."""
    npages = pg["k_pages"].shape[0]
    rows = table[torch.as_tensor(seqs, dtype=torch.long, device=table.device)].long()
    need = []
    for r, n in enumerate(seqs):
        nblk = max(int(seq_len[n]) - 1, 0) // B + 1
        need.append(rows[r, :nblk])
    need = torch.cat(need)
    uniq = torch.unique(need[(need >= 0) & (need < npages)])
    sub = {name: pg[name][uniq].cpu() for name in ("k_pages", "v_pages", "ik_pages")}
    pos = torch.searchsorted(uniq, rows.clamp(0, npages - 1))
    inb = (rows >= 0) & (rows < npages)
    hit = inb & (uniq[pos.clamp(max=len(uniq) - 1)] == rows)
    sub_table = torch.where(hit, pos, torch.full_like(pos, -1)).to(torch.int32).cpu()
    return sub, sub_table


def _paged_check(shape, seq_len, seed, share=(), bad=(), seqs=None, device="cpu",
                 extra_pages=3):
    """msa.decode_paged vs the paged oracle on the listed sequences; without
    shared or bad pages also bitwise against msa.decode on the contiguous caches."""
    msa = _msa()
    _say(f"paged decode N={shape.N} Lmax={shape.Lc} seq_len[:8]={list(seq_len[:8])} "
         f"share={list(share)} bad={list(bad)} seed={seed}")
    seq_len = np.asarray(seq_len, np.int64)
    x = synth.decode_inputs(shape, seed=seed, seq_len=np.clip(seq_len, 1, shape.Lc),
                            device=device)
    pg = synth.paginate({n: x[n] for n in ("k_cache", "v_cache", "ik_cache")}, 128, seed,
                        extra_pages=extra_pages)
    table = pg["block_table"].clone()
    for dst, src, m in share:
        table[dst, :m] = table[src, :m]
    for n, b, val in bad:
        table[n, b] = val
    g = {n: t.to(DEV) for n, t in pg.items()}
    table_d = table.to(DEV)
    q, iq = x["q"].to(DEV), x["iq"].to(DEV)
    sl = torch.tensor(seq_len.astype(np.int32), device=DEV)
    out, ids = msa.decode_paged(q, iq, g["k_pages"], g["v_pages"], g["ik_pages"], table_d, sl,
                                kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    if not share and not bad:
        kc, vc, ikc = (x[n].to(DEV) for n in ("k_cache", "v_cache", "ik_cache"))
        out_c, ids_c = msa.decode(q, iq, kc, vc, ikc, sl, kslots=shape.k, return_ids=True)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_c)
        assert torch.equal(out.view(torch.int16), out_c.view(torch.int16))
        del kc, vc, ikc
    out = out.float().cpu().numpy()
    ids = ids.cpu().numpy()
    if seqs is None:
        seqs = np.arange(shape.N)
    sub, sub_table = _compact_pages(g, table_d, seqs, seq_len)
    scale = 1.0 / math.sqrt(shape.d)
    oids, gap, oout, valid = oracle.decode_paged(x["q"][seqs], x["iq"][seqs], sub["k_pages"],
                                                 sub["v_pages"], sub["ik_pages"], sub_table,
                                                 seq_len[seqs], 128, shape.k, scale)
    vs = seqs[valid]
    for n in seqs[~valid]:
        assert (ids[n] == -1).all() and (out[n] == 0).all()
    if len(vs) == 0:
        return
    _parity.check_selection_valid(ids[vs], seq_len[vs] - 1, shape.k)
    tie, nmis = _parity.compare_ids(ids[vs], oids[valid], gap[valid])
    ref = oout[valid].copy()
    banded = 0
    if tie.any():
        # near-tie sequences: the GPU's competitors lie inside the tie band, and the
        # oracle attends the GPU's own selection
        tr = np.nonzero(tie.any(axis=1))[0]
        S = oracle.decode_paged_block_scores(x["iq"][seqs], sub["ik_pages"], sub_table,
                                             seq_len[seqs], 128, np.nonzero(valid)[0][tr])
        banded = _parity.check_near_tie_band(ids[vs[tr]], oids[valid][tr], S, seq_len[vs[tr]] - 1)
        ref[tr] = oracle.decode_paged_attend(x["q"][seqs], sub["k_pages"], sub["v_pages"],
                                             sub_table, seq_len[seqs], ids[vs[tr]], 128, scale,
                                             np.nonzero(valid)[0][tr])
    mx, mean = _parity.compare_out(out[vs], ref)
    _say(f"  -> valid {len(vs)}/{len(seqs)} near_ties {int(tie.sum())} (band checked {banded}) "
         f"mismatches {nmis} max {mx:.3e} mean {mean:.3e}")
    assert nmis == 0
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS


def test_paged_decode_small():
    shape = synth.DecodeShape(N=8, Lc=2000, H=64, G=4, d=128, dI=128, B=128, k=16)
    _paged_check(shape, np.array([1, 127, 128, 129, 2000, 1500, 640, 1999]), seed=3)


def test_paged_decode_tiny_dims():
    shape = synth.DecodeShape(N=5, Lc=4096, H=8, G=2, d=64, dI=32, B=128, k=4)
    _paged_check(shape, np.array([4096, 3000, 129, 640, 1]), seed=4, extra_pages=0)


def test_paged_decode_shared_and_bad_pages():
    """Sequences 1 and 2 reuse sequence 0's first pages (a common prefix); sequence 3
    names a page past the pool, sequence 4 a negative one, sequence 5 is longer than
    its table, sequence 6 has length 0: those four get ids -1 and zero rows."""
    shape = synth.DecodeShape(N=8, Lc=3000, H=16, G=4, d=128, dI=128, B=128, k=8)
    seq_len = np.array([3000, 2500, 1000, 2000, 700, 3000, 0, 1234])
    Lc_blocks = (shape.Lc + 127) // 128
    seq_len[5] = Lc_blocks * 128 + 1
    npages = shape.N * Lc_blocks + 2
    _paged_check(shape, seq_len, seed=5, share=[(1, 0, 12), (2, 0, 7)],
                 bad=[(3, 4, npages), (4, 0, -3)], extra_pages=2)


def test_paged_decode_full_size():
    """64 sequences x 262144 cached tokens in 131072 shuffled pages: bitwise equal to
    contiguous decode for every sequence, and the oracle on 4 of them."""
    wl = synth.WORKLOADS["decode_N64_L262144"]
    shape = wl.shape
    _paged_check(shape, np.full(shape.N, shape.Lc), seed=0, seqs=np.array([0, 21, 42, 63]),
                 device=DEV, extra_pages=0)


# --------------------------- FP8 index-key cache -----------------------------
@pytest.mark.parametrize("dI", [32, 64, 128])
def test_quantize_e4m3_vs_oracle(dI):
    """The library's cache writer gives the oracle quantizer's bytes and scales:
    rows over a wide range of magnitudes, an all-zero row, a row whose maximum is
    exactly 448 * 2^3, and rows holding every midpoint between E4M3 neighbours."""
    msa = _msa()
    rng = np.random.default_rng(dI)
    x = torch.tensor(rng.standard_normal((4099, dI)) * np.exp(rng.uniform(-30, 30, (4099, 1))),
                     dtype=torch.float32).to(torch.bfloat16)
    x[0] = 0
    x[1] = 0
    x[1, 3] = -448.0 * 8
    x[1, 4] = 17.0
    mags = oracle.e4m3_table()[:127]
    mid = torch.tensor(np.concatenate([(mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2]),
                       dtype=torch.float32)
    rows = torch.zeros((len(mid), dI))
    rows[:, 0] = mid
    rows[:, 1] = 448.0
    x = torch.cat([x, rows.to(torch.bfloat16)])
    _say(f"quantize e4m3 rows={x.shape[0]} dI={dI}")
    codes, sc = msa.quantize_idx_k_e4m3(x.to(DEV))
    torch.cuda.synchronize()
    oc, osc = oracle.quantize_e4m3_rows(x)
    bad = (codes.cpu().numpy() != oc).any(axis=1)
    _say(f"  -> rows with differing bytes {int(bad.sum())}, scales equal "
         f"{np.array_equal(sc.cpu().numpy(), osc)}")
    assert not bad.any()
    assert np.array_equal(sc.cpu().numpy(), osc)


def _fp8_decode_check(shape, seq_len, seed, seqs=None, device="cpu", spread=False,
                      scale_factor=1.0):
    """msa.decode_fp8idx vs oracle.decode_fp8idx.  The E4M3 cache is written by the
    oracle quantizer (CPU inputs) or by the torch route (inputs on the GPU); with
    `spread` each token's keys are first scaled by a random power of two, and
    `scale_factor` multiplies every stored scale (scales need not be powers of two)."""
    msa = _msa()
    _say(f"fp8 decode N={shape.N} Lmax={shape.Lc} seq_len[:8]={list(seq_len[:8])} seed={seed} "
         f"spread={spread} scale_factor={scale_factor}")
    seq_len = np.asarray(seq_len, np.int64)
    x = synth.decode_inputs(shape, seed=seed, seq_len=np.clip(seq_len, 1, shape.Lc), device=device)
    ik = x["ik_cache"]
    if spread:
        rng = np.random.default_rng(seed)
        mag = torch.tensor(np.exp2(rng.integers(-8, 9, (shape.N, shape.Lc, 1))),
                           dtype=torch.float32, device=ik.device)
        ik = (ik.float() * mag).to(torch.bfloat16)
    if device == "cpu":
        c, sc = oracle.quantize_e4m3_rows(ik)
        codes, ksc = torch.from_numpy(c), torch.from_numpy(sc)
    else:
        codes, ksc = _refs.e4m3_rows_torch(ik)
        # the torch route agrees with the oracle quantizer on a sample of rows
        rows = torch.randint(0, shape.Lc, (512,), generator=torch.Generator().manual_seed(seed))
        oc, osc = oracle.quantize_e4m3_rows(ik[0, rows.to(ik.device)].cpu())
        assert np.array_equal(codes[0, rows.to(ik.device)].cpu().numpy(), oc)
    del ik
    ksc = ksc * scale_factor
    sl = torch.tensor(seq_len.astype(np.int32), device=DEV)
    g = {n: x[n].to(DEV) for n in ("q", "iq", "k_cache", "v_cache", "ik_cache")}
    out, ids = msa.decode_fp8idx(g["q"], g["iq"], g["k_cache"], g["v_cache"], codes.to(DEV),
                                 ksc.to(DEV), sl, kslots=shape.k, return_ids=True)
    out_b, ids_b = msa.decode(g["q"], g["iq"], g["k_cache"], g["v_cache"], g["ik_cache"], sl,
                              kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    valid = (seq_len >= 1) & (seq_len <= shape.Lc)
    same = (ids == ids_b).all(dim=-1).cpu().numpy()[valid]
    out = out.float().cpu().numpy()
    ids = ids.cpu().numpy()
    if seqs is None:
        seqs = np.nonzero(valid)[0]
    scale = 1.0 / math.sqrt(shape.d)
    sub = torch.as_tensor(seqs)
    kc, vc = x["k_cache"][sub.to(x["k_cache"].device)].cpu(), x["v_cache"][sub.to(x["k_cache"].device)].cpu()
    lens = np.clip(seq_len[seqs], 1, shape.Lc)
    oids, gap, oout = oracle.decode_fp8idx(x["q"][sub.to(x["q"].device)], x["iq"][sub.to(x["q"].device)],
                                           kc, vc, codes[sub.to(codes.device)].cpu(),
                                           ksc[sub.to(ksc.device)].cpu(), lens, 128, shape.k, scale)
    pos = lens - 1
    _parity.check_selection_valid(ids[seqs], pos, shape.k)
    tie, nmis = _parity.compare_ids(ids[seqs], oids, gap)
    ref = oout.copy()
    banded = 0
    if tie.any():
        tr = np.nonzero(tie.any(axis=1))[0]
        S = oracle.decode_block_scores_fp8(x["iq"][sub.to(x["q"].device)],
                                           codes[sub.to(codes.device)].cpu(),
                                           ksc[sub.to(ksc.device)].cpu(), lens, 128, tr)
        banded = _parity.check_near_tie_band(ids[seqs[tr]], oids[tr], S, lens[tr] - 1)
        ref[tr] = oracle.decode_attend(x["q"][sub.to(x["q"].device)], kc, vc, lens, ids[seqs[tr]],
                                       128, scale, tr)
    mx, mean = _parity.compare_out(out[seqs], ref)
    _say(f"  -> near_ties {int(tie.sum())} (band checked {banded}) mismatches {nmis} "
         f"max {mx:.3e} mean {mean:.3e}; "
         f"(seq, group) selections equal to the bf16 cache's: {same.mean():.4f}")
    assert nmis == 0
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS
    for n in np.nonzero(~valid)[0]:
        assert (ids[n] == -1).all() and (out[n] == 0).all()


def test_fp8_decode_small_ragged():
    shape = synth.DecodeShape(N=8, Lc=2000, H=64, G=4, d=128, dI=128, B=128, k=16)
    _fp8_decode_check(shape, np.array([1, 127, 128, 129, 2000, 1500, 0, 2001]), seed=6)


def test_fp8_decode_spread_scales():
    shape = synth.DecodeShape(N=6, Lc=4093, H=16, G=4, d=128, dI=64, B=128, k=8)
    _fp8_decode_check(shape, np.array([4093, 3000, 129, 640, 1, 2222]), seed=7, spread=True,
                      scale_factor=1.37)


def test_fp8_decode_tiny_dims():
    shape = synth.DecodeShape(N=5, Lc=4096, H=8, G=2, d=64, dI=32, B=128, k=4)
    _fp8_decode_check(shape, np.array([4096, 3000, 129, 640, 1]), seed=8, spread=True)


def test_fp8_decode_full_size_subset():
    """64 sequences x 262144 cached tokens with an E4M3 index-key cache; oracle on 16."""
    shape = synth.WORKLOADS["decode_N64_L262144"].shape
    seqs = np.arange(0, 64, 4) + 3 * (np.arange(16) % 2)     # 0, 7, 8, 15, ..., 63
    _fp8_decode_check(shape, np.full(shape.N, shape.Lc), seed=0, seqs=seqs, device=DEV)


def _e4m3_score_band(iq, ik, codes, ksc, seq_len, B=128):
    """Per (sequence, group) of a decode batch, over the competitor blocks: the bf16
    block scores S (fp32 products of the bf16 values) and, per block, D = max over
    its tokens of |s8_t - s_t|, where s8_t is the token's score on the dequantised
    E4M3 key (scale * e4m3(byte), exact in bf16) and s_t the bf16 one.  A block
    maximum moves at most as far as its farthest token, so the E4M3 block score lies
    in [S - D, S + D].  Also the coarse per-(sequence, group) bound
    E = max_t sum_c |iq_c| |ik[t, c] - scale[t] e4m3(byte[t, c])|.  Torch on the
    inputs' device."""
    N, G = iq.shape[0], iq.shape[1]
    E = torch.zeros((N, G), dtype=torch.float64)
    S, D = [], []
    for n in range(N):
        nb = (int(seq_len[n]) - 1) // B
        T = nb * B
        if nb == 0:
            S.append(None)
            D.append(None)
            continue
        a = ik[n, :T].float()
        deq = codes[n, :T].view(torch.float8_e4m3fn).float() * ksc[n, :T, None]
        qa = iq[n].float()                                        # [G, dI]
        E[n] = ((a - deq).abs() @ qa.abs().T).amax(dim=0).double().cpu()
        s16 = a @ qa.T                                            # [T, G]
        s8 = deq @ qa.T
        S.append(s16.view(nb, B, G).amax(dim=1).T.double().cpu())            # [G, nb]
        D.append((s8 - s16).abs().view(nb, B, G).amax(dim=1).T.double().cpu())
    return E, S, D


def test_fp8_decode_band_vs_bf16_full_size():
    """The E4M3 index-key cache moves each block score by at most D (per block, from
    the bytes), so the E4M3 decode may select differently from the bf16 decode only
    among blocks whose score intervals [S - D, S + D] reach the boundary: with L15 the
    15th largest S - D and U16 the 16th largest S + D of a (sequence, group), every
    block with S - D > U16 must be selected and none with S + D < L15 may be.
    64 sequences x 262144 tokens; also reports the coarse bound E, how many blocks
    per row lie in the band, and the planted-block recall of both paths."""
    msa = _msa()
    shape = synth.WORKLOADS["decode_N64_L262144"].shape
    _say("fp8 band vs bf16, decode 64 x 262144")
    x = synth.decode_inputs(shape, seed=0, device=DEV)
    codes, ksc = _refs.e4m3_rows_torch(x["ik_cache"])
    sl = torch.tensor(np.asarray(x["seq_len"], np.int32), device=DEV)
    o8, i8 = msa.decode_fp8idx(x["q"], x["iq"], x["k_cache"], x["v_cache"], codes, ksc, sl,
                               kslots=shape.k, return_ids=True)
    ob, ib = msa.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"], sl,
                        kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    E, S, D = _e4m3_score_band(x["iq"], x["ik_cache"], codes, ksc, x["seq_len"])
    i8n, ibn = i8.cpu().numpy(), ib.cpu().numpy()
    m = shape.k - 1
    agree = 0
    band_sizes, band_picks = [], []
    for n in range(shape.N):
        nb = (int(x["seq_len"][n]) - 1) // 128
        for g in range(shape.G):
            agree += np.array_equal(i8n[n, g], ibn[n, g])
            sc, dv = S[n][g].numpy(), D[n][g].numpy()
            lo, hi = sc - dv, sc + dv
            L15 = np.sort(lo)[-m]
            U16 = np.sort(hi)[-(m + 1)]
            margin = 1e-4 * max(abs(L15), abs(U16)) + 1e-4      # fp32 accumulation
            pick = np.array([b for b in i8n[n, g] if 0 <= b < nb])
            must = np.nonzero(lo > U16 + margin)[0]
            never = hi < L15 - margin
            assert set(must.tolist()) <= set(pick.tolist()), (n, g, sorted(must), sorted(pick))
            assert not never[pick].any(), (n, g, pick[never[pick]])
            band = ~never & ~(lo > U16 + margin)
            band_sizes.append(int(band.sum()))
            band_picks.append(int(band[pick].sum()))
    rows = shape.N * shape.G
    rec = {name: np.mean([b in ids[n, g] for n in range(shape.N) for g in range(shape.G)
                          for b in x["planted"][n][g]])
           for name, ids in (("bf16", ibn), ("e4m3", i8n))}
    _say(f"  -> coarse bound E median {float(E.median()):.3f}, per-block D median "
         f"{float(np.median([d_.median().item() for d_ in D if d_ is not None])):.3f}; blocks in "
         f"the band per row: median {int(np.median(band_sizes))} (of ~2047), of which picked "
         f"{np.mean(band_picks):.1f}; identical selections {agree}/{rows}; planted-block recall "
         f"bf16 {rec['bf16']:.4f} e4m3 {rec['e4m3']:.4f}")
    assert rec["e4m3"] >= rec["bf16"] - 0.02


def test_paged_fp8_decode():
    """Paged decode over E4M3 index-key pages: the oracle on a ragged batch (with a
    bad page id and a too-long sequence), and bitwise equality with the contiguous
    E4M3 decode on the full-size workload."""
    msa = _msa()
    # ragged batch vs the oracle
    shape = synth.DecodeShape(N=6, Lc=3000, H=16, G=4, d=128, dI=128, B=128, k=8)
    seq_len = np.array([3000, 2500, 129, 1, 2000, 3000])
    x = synth.decode_inputs(shape, seed=14, seq_len=np.clip(seq_len, 1, shape.Lc))
    codes, sc = oracle.quantize_e4m3_rows(x["ik_cache"])
    x["ik8"], x["ik_scale"] = torch.from_numpy(codes), torch.from_numpy(sc)
    pg = synth.paginate(x, 128, seed=14, extra_pages=2,
                        names=("k_cache", "v_cache", "ik8", "ik_scale"))
    table = pg["block_table"].clone()
    table[4, 3] = pg["k_pages"].shape[0]               # a page past the pool
    seq_len[5] = table.shape[1] * 128 + 1              # longer than its table
    _say(f"paged fp8 decode N={shape.N} seq_len={list(seq_len)}")
    g = {n: t.to(DEV) for n, t in pg.items()}
    sl = torch.tensor(seq_len.astype(np.int32), device=DEV)
    out, ids = msa.decode_paged_fp8idx(x["q"].to(DEV), x["iq"].to(DEV), g["k_pages"],
                                       g["v_pages"], g["ik8_pages"], g["ik_scale_pages"],
                                       table.to(DEV), sl, kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    out, ids = out.float().cpu().numpy(), ids.cpu().numpy()
    scale = 1.0 / math.sqrt(shape.d)
    oids, gap, oout, valid = oracle.decode_paged_fp8idx(
        x["q"], x["iq"], pg["k_pages"], pg["v_pages"], pg["ik8_pages"], pg["ik_scale_pages"],
        table, seq_len, 128, shape.k, scale)
    assert list(valid) == [True, True, True, True, False, False]
    vs = np.nonzero(valid)[0]
    tie, nmis = _parity.compare_ids(ids[vs], oids[vs], gap[vs])
    assert not tie.any() and nmis == 0
    mx, mean = _parity.compare_out(out[vs], oout[vs])
    _say(f"  -> mismatches {nmis} max {mx:.3e} mean {mean:.3e}")
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS
    assert (ids[~valid] == -1).all() and (out[~valid] == 0).all()
    # full size: paged == contiguous, bitwise
    shape = synth.WORKLOADS["decode_N64_L262144"].shape
    x = synth.decode_inputs(shape, seed=3, device=DEV)
    x["ik8"], x["ik_scale"] = _refs.e4m3_rows_torch(x["ik_cache"])
    sl = torch.tensor(np.asarray(x["seq_len"], np.int32), device=DEV)
    o1, i1 = msa.decode_fp8idx(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik8"],
                               x["ik_scale"], sl, kslots=shape.k, return_ids=True)
    pg = synth.paginate(x, 128, seed=3, names=("k_cache", "v_cache", "ik8", "ik_scale"))
    o2, i2 = msa.decode_paged_fp8idx(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                     pg["ik8_pages"], pg["ik_scale_pages"], pg["block_table"], sl,
                                     kslots=shape.k, return_ids=True)
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_chunked_workspace_invariance():
    """A smaller workspace makes the library split the queries into several chunks;
    every row's result must be bitwise the same as with one chunk."""
    msa = _msa()
    shape = synth.PrefillShape(L=5000, H=16, G=4, d=128, dI=128, B=128, k=8)
    x = synth.prefill_inputs(shape, seed=8)
    d = {n: t.to(DEV) for n, t in x.items() if isinstance(t, torch.Tensor)}
    _say("chunked workspace invariance")
    o1, i1 = msa.prefill(d["q"], d["k"], d["v"], d["iq"], d["ik"], kslots=shape.k, return_ids=True)
    pref = msa.workspace_size("prefill", L=shape.L, H=shape.H, G=shape.G, d=shape.d, dI=shape.dI,
                              k=shape.k)
    for frac in (3, 9):
        ws = msa._workspace(pref // frac, DEV)
        o2, i2 = msa.prefill(d["q"], d["k"], d["v"], d["iq"], d["ik"], kslots=shape.k,
                             return_ids=True, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(i1, i2)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    o3 = msa.sparse_attn(d["q"], d["k"], d["v"], i1,
                         workspace=msa._workspace(msa.workspace_size(
                             "sparse_attn", L=shape.L, H=shape.H, G=shape.G, d=shape.d,
                             k=shape.k) // 4, DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
    with pytest.raises(msa.MSAError):
        msa.prefill(d["q"], d["k"], d["v"], d["iq"], d["ik"], kslots=shape.k,
                    workspace=msa._workspace(4096, DEV))


@pytest.mark.parametrize("L,H,G,d,dI,k", [(20000, 16, 4, 128, 128, 16), (9000, 8, 2, 64, 32, 4),
                                           (12000, 16, 8, 64, 64, 17), (6000, 4, 1, 64, 128, 2)])
def test_fused_selection_matches_two_kernel_path(L, H, G, d, dI, k):
    """The fused index kernel (scores, max-pool and selection in one launch, used for
    query chunks whose rows are long) gives bitwise the ids -- and so the outputs --
    of K1 + K2: a workspace for 1024-query chunks makes every chunk from query 1024
    on use it (MSA_FUSED_INDEX=1 lifts the floor on its work-group count that these
    small chunks miss), against one whole-sequence chunk served by K1 + K2; and the
    oracle on sampled rows of the chunked call."""
    msa = _msa()
    old_env = os.environ.get("MSA_FUSED_INDEX")
    os.environ["MSA_FUSED_INDEX"] = "1"
    try:
        _fused_vs_two_kernel(msa, L, H, G, d, dI, k)
    finally:
        if old_env is None:
            os.environ.pop("MSA_FUSED_INDEX", None)
        else:
            os.environ["MSA_FUSED_INDEX"] = old_env


def _fused_vs_two_kernel(msa, L, H, G, d, dI, k):
    shape = synth.PrefillShape(L=L, H=H, G=G, d=d, dI=dI, B=128, k=k)
    _say(f"fused selection L={L} H={H} G={G} d={d} dI={dI} k={k}")
    x = synth.prefill_inputs(shape, seed=9)
    dv = {n: t.to(DEV) for n, t in x.items() if isinstance(t, torch.Tensor)}
    o1, i1 = msa.prefill(dv["q"], dv["k"], dv["v"], dv["iq"], dv["ik"], kslots=k, return_ids=True)
    need = msa.workspace_size("prefill", L=1024, H=H, G=G, d=d, dI=dI, k=k)
    # the chunk size the library picks is the largest that fits: size for 1024 queries of L
    lo, hi = need, msa.workspace_size("prefill", L=L, H=H, G=G, d=d, dI=dI, k=k)
    ws = None
    for frac in (64, 32, 16, 8, 4):
        cand = max(lo, hi // frac)
        ws = msa._workspace(cand, DEV)
        try:
            o2, i2 = msa.prefill(dv["q"], dv["k"], dv["v"], dv["iq"], dv["ik"], kslots=k,
                                 return_ids=True, workspace=ws)
            break
        except msa.MSAError:
            continue
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    rows = np.unique(np.concatenate([np.arange(L - 200, L), np.random.default_rng(1).choice(L, 300, replace=False)]))
    st = _parity.prefill_rows_vs_oracle(x, rows, i2.cpu().numpy()[rows], o2.float().cpu().numpy()[rows],
                                        128, k, 1.0 / math.sqrt(d))
    _say(f"  -> {st}")
    assert st["id_mismatches"] == 0
    assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS


@pytest.mark.parametrize("frac", [10, 40])
def test_small_chunks_long_rows_on_k1(frac):
    """A workspace for a tenth (a fortieth) of the sequence gives query chunks too
    small for the fused index kernel, so chunks far from the start -- rows much
    longer than twice the chunk -- are scored by K1 + K2: the block scores must hold
    every key block.  Ids and outputs bitwise those of one whole-sequence chunk,
    for msa_prefill and msa_select_blocks."""
    msa = _msa()
    shape = synth.PrefillShape(L=40000, H=16, G=4, d=128, dI=128, B=128, k=16)
    _say(f"small chunks, long rows on K1: L={shape.L} workspace 1/{frac}")
    x = synth.prefill_inputs(shape, seed=12)
    dv = {n: t.to(DEV) for n, t in x.items() if isinstance(t, torch.Tensor)}
    o1, i1 = msa.prefill(dv["q"], dv["k"], dv["v"], dv["iq"], dv["ik"], kslots=shape.k,
                         return_ids=True)
    full = msa.workspace_size("prefill", L=shape.L, H=shape.H, G=shape.G, d=shape.d,
                              dI=shape.dI, k=shape.k)
    o2, i2 = msa.prefill(dv["q"], dv["k"], dv["v"], dv["iq"], dv["ik"], kslots=shape.k,
                         return_ids=True, workspace=msa._workspace(full // frac, DEV))
    sel_full = msa.workspace_size("select", L=shape.L, G=shape.G, dI=shape.dI, k=shape.k)
    i3 = msa.select_blocks(dv["iq"], dv["ik"], k=shape.k,
                           workspace=msa._workspace(sel_full // frac, DEV))
    torch.cuda.synchronize()
    assert torch.equal(i1, i2)
    assert torch.equal(i1, i3)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_skewed_ids_masks_and_chunking():
    """Constructed skewed ids (blocks 0-3 in nearly every row, so K4's lists of those
    blocks span many tiles) where about 5% of the rows drop block 2, some rows of
    group 1 lack all of blocks 0-3, and L is not a multiple of 128 (a short last
    query block).  Checked against the oracle on sampled rows, and bitwise against a
    run split into ~2048-query chunks."""
    msa = _msa()
    L, H, G, d, k = 24526, 16, 4, 128, 16
    shape = synth.PrefillShape(L=L, H=H, G=G, d=d, dI=128, B=128, k=k)
    _say(f"skewed ids, masks and chunking L={L} H={H} G={G}")
    x = synth.prefill_inputs(shape, seed=11, plant="none")
    ids = synth.skewed_ids(L, G, k, hot=(0, 1, 2, 3), seed=11).numpy()
    r = np.arange(L)
    drop = (r % 19 == 0) & (r // 128 >= k)
    sub = ids[drop]
    sub[sub == 2] = -1
    ids[drop] = sub
    none_rows = (r % 97 == 5) & (r // 128 >= k)          # group 1: no hot block at all
    g1 = ids[none_rows, 1]
    g1[np.isin(g1, [0, 1, 2, 3])] = -1
    ids[none_rows, 1] = g1
    dv = {n: x[n].to(DEV) for n in ("q", "k", "v")}
    idt = torch.from_numpy(ids).to(DEV)
    o1 = msa.sparse_attn(dv["q"], dv["k"], dv["v"], idt)
    full = msa.workspace_size("sparse_attn", L=L, H=H, G=G, d=d, k=k)
    o2 = msa.sparse_attn(dv["q"], dv["k"], dv["v"], idt, workspace=msa._workspace(full // 10, DEV))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    rows = np.unique(np.concatenate([np.nonzero(drop)[0][::7], np.nonzero(none_rows)[0],
                                     np.arange(L - 60, L),
                                     np.random.default_rng(2).choice(L, 700, replace=False)]))
    ref = oracle.attend(x["q"], x["k"], x["v"], ids[rows], 128, 1.0 / math.sqrt(d), rows=rows)
    mx, mean = _parity.compare_out(o1.float().cpu().numpy()[rows], ref)
    _say(f"  -> oracle on {len(rows)} rows: max {mx:.3e} mean {mean:.3e}")
    assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS


def _select_vs_oracle(iq, ik, k, rows):
    """select_blocks on the GPU and the oracle's selection for the same rows."""
    msa = _msa()
    ids = msa.select_blocks(iq.to(DEV), ik.to(DEV), k=k)
    torch.cuda.synchronize()
    S = oracle.block_scores(iq, ik, 128, rows=rows)
    oids, gap = oracle.select(S, rows, 128, k)
    got = ids.cpu().numpy()[rows]
    _parity.check_selection_valid(got, rows, k)
    return got, oids


def _constructed_select(L, w, k, rows):
    """idx_k rows w[t] * e_0 and idx_q = e_0 (G = 1, dI = 32): every token score is
    w[t] exactly, so block scores and ties are fixed by construction."""
    dI = 32
    ik = torch.zeros((L, dI), dtype=torch.bfloat16)
    ik[:, 0] = torch.as_tensor(w, dtype=torch.float32).to(torch.bfloat16)
    iq = torch.zeros((L, 1, dI), dtype=torch.bfloat16)
    iq[:, 0, 0] = 1.0
    return _select_vs_oracle(iq, ik, k, rows)


def test_select_ties_and_spread_maxima_1m():
    """L = 2^20 (8191 competitors per row at the end): (a) all scores equal, so the
    smallest ids win; (b) 128 equal maxima spread along the row (four in every 256
    blocks), so the tie between the register-held head and the streamed rest of
    the row decides the selection."""
    L, k = 1 << 20, 16
    rows = np.array([L - 1, L - 128, L // 2, 200000, 4096, 2047])
    blk = np.arange(L) // 128
    _say("select ties, L=2^20")
    got, want = _constructed_select(L, np.ones(L), k, rows)
    assert (got == want).all()
    for r, i in enumerate(rows):
        bi = i // 128
        assert got[r, 0].tolist() == list(range(min(k - 1, bi))) + [bi] + [-1] * max(0, k - bi - 1)
    _say("select spread maxima, L=2^20")
    w = np.where(blk % 256 < 4, 1000.0, -(blk % 200).astype(np.float64))
    got, want = _constructed_select(L, w, k, rows)
    assert (got == want).all()


# Row lengths (competitor counts b(i)) around the selector's layout: 4 scores per
# lane, a 1024-score register head, 256-score streaming steps, a 64-entry list.
_ADV_NB = [16, 17, 18, 31, 32, 59, 60, 61, 63, 64, 65, 127, 255, 256, 257, 511, 1023, 1024,
           1025, 1279, 1280, 1281, 2047]
_ADV_PATTERNS = ["normal", "equal", "inc", "dec", "mod3", "few", "spikes", "inc_head_dec"]


@pytest.mark.parametrize("pattern", _ADV_PATTERNS)
def test_select_constructed_block_scores(pattern):
    """Block scores fixed by construction (G = 1, dI = 32, L = 262144): one peak token
    per block at a block-dependent offset, the block's other tokens strictly lower.
    Increasing scores make every streamed score beat the running threshold (the
    candidate list is cut again and again); decreasing ones admit nothing after the
    head; equal, mod3 and few-valued scores tie heavily (the equal rows overflow the
    list from the head alone).  Ids must equal the oracle's exactly for k = 4, 16, 32."""
    nb, dI = 2048, 32
    L = nb * 128
    rng = np.random.default_rng(7)
    b = np.arange(nb)
    w = {"normal": rng.standard_normal(nb), "equal": np.ones(nb), "inc": b, "dec": -b,
         "mod3": b % 3, "few": rng.integers(0, 4, nb),
         "spikes": np.where(b % 256 < 4, 1000, -(b % 200)),
         "inc_head_dec": np.where(b < 1024, b, -b)}[pattern]
    t = np.arange(L)
    blk, off = t // 128, t % 128
    peak = off == (blk * 37) % 128
    ik = torch.zeros((L, dI), dtype=torch.bfloat16)
    iq = torch.zeros((L, 1, dI), dtype=torch.bfloat16)
    iq[:, 0, 0] = 1.0
    if pattern == "normal":
        wb = torch.as_tensor(w, dtype=torch.float32).to(torch.bfloat16).float().numpy()[blk]
        other = wb - 1.0 - (off % 5)                   # strictly below the peak after bf16 rounding
        ik[:, 0] = torch.as_tensor(np.where(peak, wb, other), dtype=torch.float32).to(torch.bfloat16)
    else:
        # integer scores as hi + lo (hi a multiple of 256, lo in [-5, 255]): both exact
        # in bf16, and their sum exact in fp32
        wb = np.asarray(w, dtype=np.int64)[blk]
        lo = np.mod(wb, 256)
        hi = wb - lo
        lo = np.where(peak, lo, lo - 1 - off % 5)
        ik[:, 0] = torch.as_tensor(hi, dtype=torch.float32).to(torch.bfloat16)
        ik[:, 1] = torch.as_tensor(lo, dtype=torch.float32).to(torch.bfloat16)
        iq[:, 0, 1] = 1.0
    rows = np.array([n * 128 + (n * 13) % 128 for n in _ADV_NB])
    for k in (4, 16, 32):
        _say(f"select constructed {pattern} k={k}")
        got, want = _select_vs_oracle(iq, ik, k, rows)
        bad = np.nonzero((got != want).any(-1))[0]
        assert len(bad) == 0, f"rows with b(i) = {[_ADV_NB[j] for j in bad]} differ"


def test_prefill_1m_hot_sampled():
    """The 1M-token skewed workload in the launch configuration the benchmark times
    (query chunks of 131072), checked on sampled rows."""
    wl = synth.WORKLOADS["prefill_L1048576_hot"]
    s = wl.shape
    _say("prefill 1M hot: generate on GPU")
    x = synth.prefill_inputs(s, seed=0, plant=wl.plant, n_plant=wl.n_plant, c=wl.c,
                             hot_blocks=wl.hot_blocks, device=DEV)
    msa = _msa()
    out, ids = msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=s.k,
                           return_ids=True)
    torch.cuda.synchronize()
    # the first two blocks, the hot blocks 0-3 (rows of their own queries), the last
    # block and 2048 uniform rows
    rows = np.unique(np.concatenate([np.arange(0, 512, 3), np.arange(s.L - 128, s.L),
                                     np.random.default_rng(3).choice(s.L, 2048, replace=False)]))
    _say(f"  oracle on {len(rows)} rows")
    # host copies: only the sampled q rows are materialised
    host = {n: x[n].cpu() for n in ("k", "v", "iq", "ik")}
    hq = torch.empty((s.L, s.H, s.d), dtype=torch.bfloat16)
    hq[torch.as_tensor(rows)] = x["q"][torch.as_tensor(rows, device=DEV)].cpu()
    host["q"] = hq
    st = _parity.prefill_rows_vs_oracle(host, rows, ids[rows].cpu().numpy(),
                                        out[rows].float().cpu().numpy(), 128, s.k,
                                        1.0 / math.sqrt(s.d))
    _say(f"  -> {st}")
    assert st["id_mismatches"] == 0
    assert st["max_abs"] < _parity.MAX_ABS and st["mean_abs"] < _parity.MEAN_ABS
    idn = ids.cpu().numpy()
    hot = (idn[128 * 5:, :, :4] == np.arange(4)).all(-1).mean()
    _say(f"  hot blocks 0-3 selected by {hot:.5f} of (query, group) rows")
    assert hot > 0.995
