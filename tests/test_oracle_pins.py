"""Pins for the CPU oracle: each check ties the oracle to something other than
itself -- a library routine in a special case the method reduces to, a
mathematical property stated on the pages, a constructed case whose answer is
fixed by construction, or brute force on tiny inputs.

Pages: "MiniMax M3 算力省 20 倍" (mizuki-eaf.pages.dev) §二 Index/Main Branch,
§三 item 4 (Local Block), §四 exp-free TopK; "MiniMax-M3上架DEVUP…" (163.com):
MSA extends GQA, per-group selection, exact attention inside selected blocks.

Every ``check_*`` takes the compiled oracle library, so the mutation test at
the bottom can run the same battery against deliberately broken copies.
"""
from __future__ import annotations

import itertools
import math
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _refs

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")

TIE = 1e-4


def _inputs(L, H, G, d, dI, B, k, seed, plant="lit"):
    s = synth.PrefillShape(L=L, H=H, G=G, d=d, dI=dI, B=B, k=k)
    return s, synth.prefill_inputs(s, seed=seed, plant=plant)


def _bf16(a) -> torch.Tensor:
    return torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16)


# --------------------------------------------------------------------------
# 1. Special case k*B >= L: every causal block is selected, so MSA is exactly
#    dense causal GQA ("MSA extends GQA", DEVUP) -> library SDPA, is_causal.
# --------------------------------------------------------------------------
def check_dense_equivalence(lib):
    for (L, H, G, d, dI, B, k, seed) in [(96, 4, 2, 16, 8, 16, 6, 0), (130, 6, 3, 8, 8, 32, 5, 1)]:
        s, x = _inputs(L, H, G, d, dI, B, k, seed)
        scale = 1.0 / math.sqrt(d)
        ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale,
                                       lib=lib)
        for i in range(L):
            bi = i // B
            for g in range(G):
                want = list(range(bi + 1)) + [-1] * (k - bi - 1)
                assert ids[i, g].tolist() == want, (i, g, ids[i, g])
        ref = _refs.sdpa_causal(x["q"], x["k"], x["v"], scale).numpy()
        assert np.abs(out - ref).max() < 1e-9


# --------------------------------------------------------------------------
# 2. Special case k = 1: only the query's own block -> block-diagonal causal
#    attention -> library SDPA with that mask.
# --------------------------------------------------------------------------
def check_local_only(lib):
    L, H, G, d, dI, B = 100, 4, 2, 16, 8, 16
    s, x = _inputs(L, H, G, d, dI, B, 1, 2)
    scale = 0.3
    ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, 1, scale, lib=lib)
    assert (ids[:, :, 0] == (np.arange(L) // B)[:, None]).all()
    blk = torch.arange(L) // B
    m = (blk[:, None] == blk[None, :]) & torch.tril(torch.ones(L, L, dtype=torch.bool))
    ref = _refs.sdpa_masked(x["q"], x["k"], x["v"], m[None].expand(H, L, L), scale).numpy()
    assert np.abs(out - ref).max() < 1e-9


# --------------------------------------------------------------------------
# 3. Main branch for an arbitrary selection equals library attention with
#    the mask "block selected by the query's group, and t <= i".
# --------------------------------------------------------------------------
def check_masked_attention(lib):
    for (L, H, G, d, dI, B, k, seed) in [(200, 8, 2, 16, 8, 16, 4, 3), (160, 6, 3, 24, 8, 32, 3, 4)]:
        s, x = _inputs(L, H, G, d, dI, B, k, seed)
        scale = 1.0 / math.sqrt(d)
        ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale,
                                       lib=lib)
        mask = _refs.mask_from_ids(ids, L, B, H, G)
        ref = _refs.sdpa_masked(x["q"], x["k"], x["v"], mask, scale).numpy()
        assert np.abs(out - ref).max() < 1e-9
        # the same holds for ids that did not come from the index branch
        rng = np.random.default_rng(seed)
        ids2 = np.full_like(ids, -1)
        for i in range(L):
            bi = i // B
            for g in range(G):
                extra = rng.choice(bi, size=min(k - 1, bi), replace=False) if bi else []
                ch = sorted(list(extra) + [bi])
                ids2[i, g, :len(ch)] = ch
        out2 = oracle.attend(x["q"], x["k"], x["v"], ids2, B, scale, lib=lib)
        ref2 = _refs.sdpa_masked(x["q"], x["k"], x["v"],
                                 _refs.mask_from_ids(ids2, L, B, H, G), scale).numpy()
        assert np.abs(out2 - ref2).max() < 1e-9


# --------------------------------------------------------------------------
# 4. exp-free selection == selection after softmax (softmax keeps order;
#    "MiniMax M3 算力省 20 倍" §四 exp-free TopK): softmax over the causal token
#    scores, max-pool of probabilities, library top-k.
# --------------------------------------------------------------------------
def check_exp_free(lib):
    for (L, G, dI, B, k, seed, plant) in [(384, 2, 16, 16, 5, 5, "lit"), (512, 3, 8, 32, 4, 6, "none"),
                                          (256, 2, 32, 8, 6, 7, "hot")]:
        s, x = _inputs(L, G, G, 8, dI, B, k, seed, plant)
        S = oracle.block_scores(x["iq"], x["ik"], B, lib=lib)
        ids, gap = oracle.select(S, np.arange(L), B, k, lib=lib)
        ref = _refs.softmax_pool_topk(x["iq"], x["ik"], B, k)
        ok = gap >= TIE
        assert ok.mean() > 0.9
        assert (ids[ok] == ref[ok]).all()


# --------------------------------------------------------------------------
# 5. Constructed cases: idx-K rows are multiples of basis vectors, so every
#    token score, every block maximum and hence the selection are fixed by
#    construction (no dot product is evaluated by the test).
# --------------------------------------------------------------------------
def _constructed(seed):
    """G=3 groups, dI=4, B=8, L=96 (12 blocks), k=4.
    ik[t] = w[t] * e_0 + z[t] * e_1.  Group 0 uses iq = e_0 (score w),
    group 1 uses iq = -e_0 (score -w), group 2 uses iq = 2 e_1 (score 2 z)."""
    rng = np.random.default_rng(seed)
    L, G, dI, B, k = 96, 3, 4, 8, 4
    nb = L // B
    # block maxima: distinct integers; the max sits at a random position
    peak_w = rng.permutation(nb) + 20          # max of w per block (group 0 ranks)
    low_w = -(rng.permutation(nb) + 20)        # min of w per block (group 1 ranks -w)
    peak_z = rng.permutation(nb) + 20
    w = np.zeros(L)
    z = np.zeros(L)
    for b in range(nb):
        vals = rng.integers(-8, 9, size=B).astype(float)   # filler strictly inside (-20, 20)
        pw, pl = rng.choice(B, size=2, replace=False)
        vals[pw] = peak_w[b]
        vals[pl] = low_w[b]
        w[b * B:(b + 1) * B] = vals
        zv = rng.integers(-8, 9, size=B).astype(float)
        zv[rng.integers(B)] = peak_z[b]
        z[b * B:(b + 1) * B] = zv
    ik = np.zeros((L, dI))
    ik[:, 0] = w
    ik[:, 1] = z
    iq = np.zeros((L, G, dI))
    iq[:, 0, 0] = 1.0
    iq[:, 1, 0] = -1.0
    iq[:, 2, 1] = 2.0
    # expected: per group a rank value per block (larger = better), only blocks < b(i)
    rank = np.stack([peak_w, -low_w, 2 * peak_z])          # [G, nb] block maxima by construction
    return L, G, dI, B, k, ik, iq, rank, w, z


def check_constructed(lib):
    for seed in range(3):
        L, G, dI, B, k, ik, iq, rank, w, z = _constructed(seed)
        S = oracle.block_scores(_bf16(iq), _bf16(ik), B, lib=lib)
        nb = L // B
        for i in range(L):
            bi = i // B
            for g in range(G):
                # competitors' block scores are the constructed maxima
                assert np.array_equal(S[i, g, :bi], rank[g, :bi].astype(np.float32)), (i, g)
                # the own block is scored over the causal window t <= i only
                t = np.arange(bi * B, i + 1)
                tok = [w[t], -w[t], 2 * z[t]][g]
                assert S[i, g, bi] == np.float32(tok.max()), (i, g)
                assert np.all(np.isneginf(S[i, g, bi + 1:]))
        ids, gap = oracle.select(S, np.arange(L), B, k, lib=lib)
        for i in range(L):
            bi = i // B
            for g in range(G):
                order = np.argsort(-rank[g, :bi], kind="stable")[:k - 1]
                want = sorted(list(order) + [bi])
                want += [-1] * (k - len(want))
                assert ids[i, g].tolist() == want, (seed, i, g, ids[i, g], want)


def check_tie_break(lib):
    """Equal block scores: the smaller block id wins (reading where the pages
    are silent).  Every token score equals 1, so all blocks tie."""
    L, G, dI, B, k = 64, 1, 2, 8, 3
    ik = np.zeros((L, dI))
    ik[:, 0] = 1.0
    iq = np.zeros((L, G, dI))
    iq[:, 0, 0] = 1.0
    S = oracle.block_scores(_bf16(iq), _bf16(ik), B, lib=lib)
    ids, gap = oracle.select(S, np.arange(L), B, k, lib=lib)
    for i in range(L):
        bi = i // B
        want = sorted(set(list(range(min(k - 1, bi))) + [bi]))
        assert ids[i, 0].tolist() == want + [-1] * (k - len(want))
        if bi > k - 1:
            assert gap[i, 0] == 0.0


# --------------------------------------------------------------------------
# 6. Brute force on tiny inputs: explicit token-score loops, pooled block
#    scores, and the selection as the k-1-subset of competitors with the
#    largest total score (equivalent to top-(k-1) when scores are distinct),
#    then attention with explicit per-token weights.
# --------------------------------------------------------------------------
def _brute(q, kk, vv, iq, ik, B, k, scale):
    q, kk, vv, iq, ik = (_refs.f64(a).numpy() for a in (q, kk, vv, iq, ik))
    L, H, d = q.shape
    G = kk.shape[1]
    r = H // G
    ids = np.full((L, G, k), -1, np.int32)
    out = np.zeros((L, H, d))
    for i in range(L):
        bi = i // B
        for g in range(G):
            tok = {t: float(np.dot(iq[i, g], ik[t])) for t in range(i + 1)}
            blk = {}
            for t, sc in tok.items():
                blk[t // B] = max(blk.get(t // B, -np.inf), sc)
            comp = [b for b in range(bi)]
            m = min(k - 1, len(comp))
            best, best_sum = (), -np.inf
            for sub in itertools.combinations(comp, m):
                tot = sum(np.float32(blk[b]) for b in sub)
                if tot > best_sum:
                    best, best_sum = sub, tot
            ch = sorted(list(best) + [bi])
            ids[i, g, :len(ch)] = ch
            toks = [t for t in range(i + 1) if t // B in ch]
            for hh in range(g * r, (g + 1) * r):
                z = np.array([scale * np.dot(q[i, hh], kk[t, g]) for t in toks])
                p = np.exp(z - z.max())
                p /= p.sum()
                out[i, hh] = sum(p[u] * vv[t, g] for u, t in enumerate(toks))
    return ids, out


def check_brute_force(lib):
    for (L, H, G, d, dI, B, k, seed) in [(40, 4, 2, 8, 4, 4, 3, 8), (48, 2, 1, 4, 4, 8, 2, 9),
                                         (36, 6, 3, 4, 8, 4, 1, 10)]:
        s, x = _inputs(L, H, G, d, dI, B, k, seed)
        scale = 1.0 / math.sqrt(d)
        ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale,
                                       lib=lib)
        bids, bout = _brute(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale)
        ok = gap >= TIE
        assert (ids[ok] == bids[ok]).all()
        okrow = np.repeat(ok, H // G, axis=1)
        assert np.abs(out - bout)[okrow].max() < 1e-9


# --------------------------------------------------------------------------
# 7. Invariants of every selection ("MiniMax M3 算力省 20 倍" §二, §三 item 4):
#    own block present, ids unique/ascending/in range, count = min(k, b(i)+1).
# --------------------------------------------------------------------------
def assert_selection_invariants(ids: np.ndarray, rows: np.ndarray, B: int, k: int):
    for r, i in enumerate(rows):
        bi = int(i) // B
        n = min(k, bi + 1)
        for g in range(ids.shape[1]):
            row = ids[r, g]
            assert (row[n:] == -1).all(), (i, g, row)
            v = row[:n]
            assert (v >= 0).all() and (v <= bi).all(), (i, g, row)
            assert (np.diff(v) > 0).all(), (i, g, row)
            assert bi in v, (i, g, row)


def check_invariants(lib):
    for (L, G, dI, B, k, seed) in [(1000, 2, 16, 16, 5, 11), (777, 4, 8, 32, 3, 12)]:
        s, x = _inputs(L, G, G, 8, dI, B, k, seed)
        S = oracle.block_scores(x["iq"], x["ik"], B, lib=lib)
        ids, gap = oracle.select(S, np.arange(L), B, k, lib=lib)
        assert_selection_invariants(ids, np.arange(L), B, k)


# --------------------------------------------------------------------------
# 8. Property tests: scale invariance, within-block permutation, planted block.
# --------------------------------------------------------------------------
def check_properties(lib):
    L, H, G, d, dI, B, k = 256, 4, 2, 16, 16, 16, 4
    s, x = _inputs(L, H, G, d, dI, B, k, 13)
    scale = 1.0 / math.sqrt(d)
    ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale, lib=lib)
    # (a) doubling idx-Q (exact in bf16) changes no selection
    ids2, gap2, _ = oracle.prefill(x["q"], x["k"], x["v"], x["iq"] * 2, x["ik"], B, k, scale,
                                   lib=lib)
    assert (ids2 == ids).all()
    # (b) permuting the tokens inside block j leaves every later row unchanged
    j = 5
    perm = torch.randperm(B, generator=torch.Generator().manual_seed(0)) + j * B
    y = {n: t.clone() for n, t in x.items() if isinstance(t, torch.Tensor)}
    for n in ("k", "v", "ik"):
        y[n][j * B:(j + 1) * B] = x[n][perm]
    ids3, gap3, out3 = oracle.prefill(y["q"], y["k"], y["v"], y["iq"], y["ik"], B, k, scale,
                                      lib=lib)
    later = np.arange(L) >= (j + 1) * B
    assert (ids3[later] == ids[later]).all()
    assert np.abs(out3[later] - out[later]).max() < 1e-12
    # (c) a planted block with a large score along each group's query direction
    #     is selected by every row that can select it
    j = 3
    u = x["iq"].float().mean(0)                                   # [G, dI]
    y = {n: t.clone() for n, t in x.items() if isinstance(t, torch.Tensor)}
    y["iq"] = (x["iq"].float() + 3.0 * u.sign()[None]).to(torch.bfloat16)
    y["ik"][j * B:(j + 1) * B] = (50.0 * u.sign().sum(0).sign())[None].to(torch.bfloat16)
    ids4, _, _ = oracle.prefill(y["q"], y["k"], y["v"], y["iq"], y["ik"], B, k, scale, lib=lib)
    rows = np.arange(L)[np.arange(L) // B > j]
    assert all(j in ids4[i, g] for i in rows for g in range(G))


# --------------------------------------------------------------------------
# 9. Prefix consistency and decode == last prefill row.
# --------------------------------------------------------------------------
def check_prefix_and_decode(lib):
    L, H, G, d, dI, B, k = 300, 4, 2, 16, 8, 16, 4
    s, x = _inputs(L, H, G, d, dI, B, k, 14)
    scale = 1.0 / math.sqrt(d)
    ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale, lib=lib)
    Lp = 173
    idsp, gapp, outp = oracle.prefill(x["q"][:Lp], x["k"][:Lp], x["v"][:Lp], x["iq"][:Lp],
                                      x["ik"][:Lp], B, k, scale, lib=lib)
    assert (idsp == ids[:Lp]).all()
    assert np.array_equal(outp, out[:Lp])
    # decode: sequence n holds the prefill tensors; its query is token seq_len-1
    seq_len = np.array([300, 1, 16, 17, 255], np.int64)
    N = len(seq_len)
    qd = torch.stack([x["q"][sl - 1] for sl in seq_len])
    iqd = torch.stack([x["iq"][sl - 1] for sl in seq_len])
    kc = x["k"][None].expand(N, L, G, d).contiguous()
    vc = x["v"][None].expand(N, L, G, d).contiguous()
    ikc = x["ik"][None].expand(N, L, dI).contiguous()
    idsd, gapd, outd = oracle.decode(qd, iqd, kc, vc, ikc, seq_len, B, k, scale, lib=lib)
    for n, sl in enumerate(seq_len):
        assert (idsd[n] == ids[sl - 1]).all()
        assert np.array_equal(outd[n], out[sl - 1])


def check_decode_distinct_sequences(lib):
    """Decode over caches that differ per sequence (three independently seeded
    sequences, each cache padded to Lmax with unrelated values past its length)
    equals each sequence's own prefill at its last token, bit for bit."""
    B, k, H, G, d, dI = 16, 4, 4, 2, 16, 8
    lens = [150, 77, 200]
    Lmax = 200
    scale = 1.0 / math.sqrt(d)
    seqs = [_inputs(L, H, G, d, dI, B, k, 30 + n)[1] for n, L in enumerate(lens)]
    pad = _inputs(Lmax, H, G, d, dI, B, k, 99)[1]
    def cache(name):
        out = []
        for x, L in zip(seqs, lens):
            out.append(torch.cat([x[name], pad[name][L:]]))
        return torch.stack(out)
    qd = torch.stack([x["q"][L - 1] for x, L in zip(seqs, lens)])
    iqd = torch.stack([x["iq"][L - 1] for x, L in zip(seqs, lens)])
    ids, gap, out = oracle.decode(qd, iqd, cache("k"), cache("v"), cache("ik"),
                                  np.array(lens, np.int64), B, k, scale, lib=lib)
    for n, (x, L) in enumerate(zip(seqs, lens)):
        pid, pgap, pout = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale,
                                         rows=np.array([L - 1]), lib=lib)
        assert (ids[n] == pid[0]).all()
        assert np.array_equal(out[n], pout[0])


def _distinct_decode_case():
    """Three independently seeded sequences in caches padded to Lmax with unrelated
    values past each length (the setting of check_decode_distinct_sequences)."""
    B, k, H, G, d, dI = 16, 4, 4, 2, 16, 8
    lens = [150, 77, 200]
    Lmax = 200
    seqs = [_inputs(L, H, G, d, dI, B, k, 30 + n)[1] for n, L in enumerate(lens)]
    pad = _inputs(Lmax, H, G, d, dI, B, k, 99)[1]
    cache = {name: torch.stack([torch.cat([x[name], pad[name][L:]]) for x, L in zip(seqs, lens)])
             for name in ("k", "v", "ik")}
    qd = torch.stack([x["q"][L - 1] for x, L in zip(seqs, lens)])
    iqd = torch.stack([x["iq"][L - 1] for x, L in zip(seqs, lens)])
    return B, k, d, lens, seqs, cache, qd, iqd


def _random_valid_ids(rng, pos, G, k, B):
    """Arbitrary valid selections (not from the index branch): the own block plus up
    to k-1 distinct earlier blocks, ascending, -1 padded."""
    ids = np.full((len(pos), G, k), -1, np.int32)
    for r, i in enumerate(pos):
        bi = int(i) // B
        for g in range(G):
            m = int(rng.integers(0, min(k - 1, bi) + 1))
            ch = sorted(list(rng.choice(bi, size=m, replace=False)) + [bi]) if bi else [0]
            ids[r, g, :len(ch)] = ch
    return ids


def check_decode_attend(lib):
    """The decode main branch on given ids (what the parity tests attend on near-tie
    rows) is the prefill main branch of each sequence's own data at its last token:
    with the ids decode selected it reproduces decode bit for bit, and with arbitrary
    valid ids it equals oracle.attend on that sequence's row L-1 (pinned to library
    SDPA by check_masked_attention), for sequences listed in any order."""
    B, k, d, lens, seqs, cache, qd, iqd = _distinct_decode_case()
    scale = 1.0 / math.sqrt(d)
    lens_a = np.array(lens, np.int64)
    ids, gap, out = oracle.decode(qd, iqd, cache["k"], cache["v"], cache["ik"], lens_a, B, k,
                                  scale, lib=lib)
    att = oracle.decode_attend(qd, cache["k"], cache["v"], lens_a, ids, B, scale, [0, 1, 2],
                               lib=lib)
    assert np.array_equal(att, out)
    rng = np.random.default_rng(5)
    G = iqd.shape[1]
    order = [2, 0, 1]
    rids = _random_valid_ids(rng, lens_a[order] - 1, G, k, B)
    att2 = oracle.decode_attend(qd, cache["k"], cache["v"], lens_a, rids, B, scale, order,
                                lib=lib)
    for r, n in enumerate(order):
        x, L = seqs[n], lens[n]
        ref = oracle.attend(x["q"], x["k"], x["v"], rids[r:r + 1], B, scale,
                            rows=np.array([L - 1]), lib=lib)
        assert np.array_equal(att2[r], ref[0]), (n, L)


def check_decode_block_scores(lib):
    """Decode block scores (what the parity tests' near-tie band check reads) are the
    prefill block scores of each sequence's own data at its last token, -inf past the
    own block; the selection on them is decode's.  Over an E4M3 cache with power-of-two
    scales they equal the scores of the dequantised keys; over pages they equal the
    contiguous cache's."""
    B, k, d, lens, seqs, cache, qd, iqd = _distinct_decode_case()
    lens_a = np.array(lens, np.int64)
    order = [1, 2, 0]
    S = oracle.decode_block_scores(iqd, cache["ik"], lens_a, B, order, lib=lib)
    for r, n in enumerate(order):
        x, L = seqs[n], lens[n]
        ref = oracle.block_scores(x["iq"], x["ik"], B, rows=np.array([L - 1]), lib=lib)[0]
        nb = ref.shape[1]
        assert np.array_equal(S[r, :, :nb], ref), (n, L)
        assert np.isneginf(S[r, :, nb:]).all()
    ids, gap, _ = oracle.decode(qd, iqd, cache["k"], cache["v"], cache["ik"], lens_a, B, k,
                                1.0, seqs=order, lib=lib)
    sids, sgap = oracle.select(S, lens_a[order] - 1, B, k, lib=lib)
    assert np.array_equal(sids, ids) and np.array_equal(sgap, gap)
    # E4M3 cache with power-of-two scales == the dequantised bf16 keys
    rng = np.random.default_rng(17)
    mag = torch.tensor(np.exp2(rng.integers(-5, 6, (3, cache["ik"].shape[1], 1))),
                       dtype=torch.float32)
    ikx = (cache["ik"].float() * mag).to(torch.bfloat16)
    codes, sc = oracle.quantize_e4m3_rows(ikx, lib)
    table = oracle.e4m3_table(lib)
    deq = _bf16(table[codes] * sc[..., None])
    S8 = oracle.decode_block_scores_fp8(iqd, codes, sc, lens_a, B, order, lib=lib)
    Sd = oracle.decode_block_scores(iqd, deq, lens_a, B, order, lib=lib)
    assert np.array_equal(S8, Sd)
    # pages laid out by an independent permutation == the contiguous cache
    pg = synth.paginate({"ik_cache": cache["ik"]}, B, seed=8, extra_pages=3, names=("ik_cache",))
    Sp = oracle.decode_paged_block_scores(iqd, pg["ik_pages"], pg["block_table"], lens_a, B,
                                          order, lib=lib)
    assert np.array_equal(Sp, S)


def check_paged_attend(lib):
    """The paged decode main branch on given ids is the paged decode's own when fed
    its ids (shuffled pages, and pages shared between sequences), and the contiguous
    decode main branch on the caches the table spells out for arbitrary valid ids."""
    B, k = 16, 4
    sh = synth.DecodeShape(N=4, Lc=150, H=4, G=2, d=16, dI=8, B=B, k=k)
    seq_len = np.array([150, 40, 97, 64], np.int64)
    x = synth.decode_inputs(sh, seed=22, seq_len=seq_len)
    pg = synth.paginate(x, B, seed=22, extra_pages=4)
    scale = 1.0 / math.sqrt(sh.d)
    for share in (False, True):
        table = pg["block_table"].clone()
        if share:
            table[2, :3] = table[0, :3]
        ids, _, out, valid = oracle.decode_paged(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                                 pg["ik_pages"], table, seq_len, B, k, scale,
                                                 lib=lib)
        assert valid.all()
        att = oracle.decode_paged_attend(x["q"], pg["k_pages"], pg["v_pages"], table, seq_len,
                                         ids, B, scale, np.arange(sh.N), lib=lib)
        assert np.array_equal(att, out), share
    rng = np.random.default_rng(9)
    order = np.array([3, 1, 0])
    rids = _random_valid_ids(rng, seq_len[order] - 1, sh.G, k, B)
    att2 = oracle.decode_paged_attend(x["q"], pg["k_pages"], pg["v_pages"], pg["block_table"],
                                      seq_len, rids, B, scale, order, lib=lib)
    ref = oracle.decode_attend(x["q"], x["k_cache"], x["v_cache"], seq_len, rids, B, scale,
                               order, lib=lib)
    assert np.array_equal(att2, ref)


def check_gap_definition(lib):
    """The near-tie gap of a row is |a - c| / max(|a|, |c|) for a = the score of the
    last selected competitor and c = the best unselected one (0 when both are 0),
    and +inf when every competitor is selected; constructed block scores."""
    B, k, nb = 4, 4, 12
    base = np.array([5, 9, 1, 7, 3, 8, 2, 6, 4, 0], np.float32)
    S = np.full((3, 5, nb), -np.inf, np.float32)
    S[0, 0, :10] = base                      # picks 9, 8, 7; next 6
    S[0, 1, :10] = -base                     # picks 0, -1, -2; next -3
    S[0, 2, :10] = [1, 1, 1, 1, 1, 0, 0, 0, 0, 0]   # ties: picks blocks 0-2; next 1
    S[0, 3, :10] = [0.5, -0.5, 3, 2, -4, -5, -6, -7, -8, -9]   # picks 3, 2, .5; next -.5
    S[0, 4, :10] = 0.0
    S[1, :, :2] = [[1, 2]] * 5               # row with b(i) = 2: every competitor taken
    S[2, :, :10] = base
    rows = np.array([10 * B + 1, 2 * B + 3, 10 * B + 3])
    ids, gap = oracle.select(S, rows, B, k, lib=lib)
    assert ids[0, 0].tolist() == [1, 3, 5, 10]
    assert ids[0, 1].tolist() == [2, 6, 9, 10]
    assert ids[0, 2].tolist() == [0, 1, 2, 10]
    assert ids[0, 3].tolist() == [0, 2, 3, 10]
    expect = [1.0 / 7.0, 1.0 / 3.0, 0.0, 2.0, 0.0]
    for g, e in enumerate(expect):
        assert abs(float(gap[0, g]) - e) < 1e-6, (g, gap[0, g], e)
    assert np.isinf(gap[1]).all() and (ids[1, :, :3] == [0, 1, 2]).all()
    assert abs(float(gap[2, 0]) - 1.0 / 7.0) < 1e-6


# --------------------------------------------------------------------------
# 10. Paged decode ("MiniMax M3 的采用瓶颈…" §对建设者的影响: paged MSA decode) is
#     decode on the cache that the block table spells out: pages laid out by an
#     independent seeded permutation (synth.paginate) must give the contiguous
#     decode bit for bit; a table that points two sequences at the same pages must
#     give decode on caches whose prefixes were copied in contiguous form; a bad
#     page id or length marks the sequence invalid.
# --------------------------------------------------------------------------
def check_paged_decode(lib):
    B, k = 16, 4
    sh = synth.DecodeShape(N=4, Lc=150, H=4, G=2, d=16, dI=8, B=B, k=k)
    seq_len = np.array([150, 1, 97, 64], np.int64)
    x = synth.decode_inputs(sh, seed=21, seq_len=seq_len)
    pg = synth.paginate(x, B, seed=21, extra_pages=5)
    scale = 1.0 / math.sqrt(sh.d)
    ids, gap, out = oracle.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"],
                                  seq_len, B, k, scale, lib=lib)
    idsp, gapp, outp, valid = oracle.decode_paged(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                                  pg["ik_pages"], pg["block_table"], seq_len, B,
                                                  k, scale, lib=lib)
    assert valid.all()
    assert np.array_equal(idsp, ids) and np.array_equal(outp, out)
    # sequence 2 shares sequence 0's first 3 pages
    table = pg["block_table"].clone()
    table[2, :3] = table[0, :3]
    kc, vc, ikc = x["k_cache"].clone(), x["v_cache"].clone(), x["ik_cache"].clone()
    kc[2, :3 * B], vc[2, :3 * B], ikc[2, :3 * B] = kc[0, :3 * B], vc[0, :3 * B], ikc[0, :3 * B]
    ids2, _, out2 = oracle.decode(x["q"], x["iq"], kc, vc, ikc, seq_len, B, k, scale, lib=lib)
    idsp2, _, outp2, _ = oracle.decode_paged(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                             pg["ik_pages"], table, seq_len, B, k, scale, lib=lib)
    assert np.array_equal(idsp2, ids2) and np.array_equal(outp2, out2)
    assert not np.array_equal(out2[2], out[2])
    # a page id out of range, a length past the table: invalid, ids -1, zero output
    npages = pg["k_pages"].shape[0]
    table[3, 1] = npages
    bad_len = seq_len.copy()
    bad_len[1] = table.shape[1] * B + 1
    idsp3, _, outp3, valid3 = oracle.decode_paged(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                                  pg["ik_pages"], table, bad_len, B, k, scale,
                                                  lib=lib)
    assert list(valid3) == [True, False, True, False]
    assert (idsp3[[1, 3]] == -1).all() and not outp3[[1, 3]].any()
    # an entry past the sequence's last block is never read
    table[0, -1] = -7
    short = seq_len.copy()
    short[0] = (table.shape[1] - 1) * B
    _, _, _, valid4 = oracle.decode_paged(x["q"], x["iq"], pg["k_pages"], pg["v_pages"],
                                          pg["ik_pages"], table, short, B, k, scale, lib=lib)
    assert valid4[0]


# --------------------------------------------------------------------------
# 11. FP8 index-key cache.  E4M3 is the OCP 8-bit floating point encoding; the
#     library routine torch.float8_e4m3fn implements the same encoding, so it
#     pins the oracle's byte decoding (all 256 bytes) and its round-to-nearest-
#     even quantizer (random rows over a wide range of magnitudes, every midpoint
#     between neighbouring values).  With power-of-two scales the dequantised keys
#     are exact in bf16, so FP8 decode must equal bf16 decode on them; a scale
#     other than a power of two multiplies the token's score.
# --------------------------------------------------------------------------
def _e4m3_ref(x):
    return torch.as_tensor(x, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def check_e4m3(lib):
    table = oracle.e4m3_table(lib)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(table), np.isnan(ref))
    assert np.array_equal(table[~np.isnan(table)], ref[~np.isnan(ref)])
    rng = np.random.default_rng(3)
    x = torch.tensor(rng.standard_normal((300, 64)) * np.exp(rng.uniform(-25, 25, (300, 1))),
                     dtype=torch.float32).to(torch.bfloat16)
    x[0] = 0
    x[1] = x[1] / x[1].abs().max().float().item() * 100
    x[1, 7] = -448 * 2.0 ** 5            # amax exactly 448 * 2^5 -> scale 2^5
    codes, sc = oracle.quantize_e4m3_rows(x, lib)
    xf = x.double().numpy()
    amax = np.abs(xf).max(axis=1)
    assert sc[0] == 1.0 and sc[1] == 32.0
    assert (amax <= 448.0 * sc).all() and (amax[2:] > 224.0 * sc[2:]).all()
    assert np.all(np.log2(sc) == np.round(np.log2(sc)))
    assert np.array_equal(codes, _e4m3_ref(xf / sc[:, None]))
    mags = table[:127]
    mid = (mags[:-1] + mags[1:]) / 2
    rows = np.zeros((2 * len(mid), 2))
    rows[:, 0] = np.concatenate([mid, -mid])
    rows[:, 1] = 448.0
    codes2, sc2 = oracle.quantize_e4m3_rows(_bf16(rows), lib)
    assert (sc2 == 1.0).all()
    assert np.array_equal(codes2, _e4m3_ref(rows))


def check_fp8_decode(lib):
    B, k = 16, 4
    sh = synth.DecodeShape(N=4, Lc=200, H=4, G=2, d=16, dI=8, B=B, k=k)
    seq_len = np.array([200, 1, 97, 150], np.int64)
    x = synth.decode_inputs(sh, seed=23, seq_len=seq_len)
    # token magnitudes spread over 2^-6 .. 2^6 so the per-token scales differ
    rng = np.random.default_rng(23)
    mag = torch.tensor(np.exp2(rng.integers(-6, 7, (sh.N, sh.Lc, 1))), dtype=torch.float32)
    ikx = (x["ik_cache"].float() * mag).to(torch.bfloat16)
    codes, sc = oracle.quantize_e4m3_rows(ikx, lib)
    assert len(np.unique(sc)) > 5
    table = oracle.e4m3_table(lib)
    deq = _bf16(table[codes] * sc[..., None])
    assert np.array_equal(deq.double().numpy(), table[codes] * sc[..., None])   # exact in bf16
    scale = 1.0 / math.sqrt(sh.d)
    ids8, gap8, out8 = oracle.decode_fp8idx(x["q"], x["iq"], x["k_cache"], x["v_cache"], codes,
                                            sc, seq_len, B, k, scale, lib=lib)
    ids, gap, out = oracle.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], deq, seq_len, B,
                                  k, scale, lib=lib)
    assert np.array_equal(ids8, ids) and np.array_equal(out8, out)
    np.testing.assert_array_equal(gap8, gap)
    # a non-power-of-two scale multiplies the score: two blocks holding the same
    # bytes, the one with the larger scale wins (the query's dot product is > 0)
    N1, L1, dI = 1, 5 * B, 8
    q1 = torch.zeros((1, 2, 4), dtype=torch.bfloat16)
    iq1 = _bf16(np.ones((1, 1, dI)))
    kv1 = torch.zeros((1, L1, 1, 4), dtype=torch.bfloat16)
    ik8 = np.full((1, L1, dI), 0x30, np.uint8)          # e4m3 0x30 = 1.0
    ks = np.ones((1, L1), np.float32)
    ks[0, 1 * B:2 * B] = 1.25
    ks[0, 3 * B:4 * B] = 1.5
    ids1, _, _ = oracle.decode_fp8idx(q1, iq1, kv1, kv1, ik8, ks, [L1], B, 2, 1.0, lib=lib)
    assert list(ids1[0, 0]) == [3, 4]
    ks[0, 3 * B + 7] = 0.5                                 # max over the block still 1.5
    ks[0, 1 * B + 9] = 1.75
    ids2, _, _ = oracle.decode_fp8idx(q1, iq1, kv1, kv1, ik8, ks, [L1], B, 2, 1.0, lib=lib)
    assert list(ids2[0, 0]) == [1, 4]


def check_paged_fp8_decode(lib):
    """Paged decode over E4M3 index-key pages equals the contiguous E4M3 decode on
    the caches an independent seeded page permutation scatters."""
    B, k = 16, 4
    sh = synth.DecodeShape(N=3, Lc=170, H=4, G=2, d=16, dI=8, B=B, k=k)
    seq_len = np.array([170, 33, 120], np.int64)
    x = synth.decode_inputs(sh, seed=27, seq_len=seq_len)
    codes, sc = oracle.quantize_e4m3_rows(x["ik_cache"], lib)
    x["ik8"], x["ik_scale"] = torch.from_numpy(codes), torch.from_numpy(sc * 1.5)
    pg = synth.paginate(x, B, seed=27, extra_pages=2,
                        names=("k_cache", "v_cache", "ik8", "ik_scale"))
    scale = 1.0 / math.sqrt(sh.d)
    ids, gap, out = oracle.decode_fp8idx(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik8"],
                                         x["ik_scale"], seq_len, B, k, scale, lib=lib)
    idsp, gapp, outp, valid = oracle.decode_paged_fp8idx(
        x["q"], x["iq"], pg["k_pages"], pg["v_pages"], pg["ik8_pages"], pg["ik_scale_pages"],
        pg["block_table"], seq_len, B, k, scale, lib=lib)
    assert valid.all()
    assert np.array_equal(idsp, ids) and np.array_equal(outp, out)


PINS = [check_dense_equivalence, check_local_only, check_masked_attention, check_exp_free,
        check_constructed, check_tie_break, check_brute_force, check_invariants,
        check_properties, check_prefix_and_decode, check_decode_distinct_sequences,
        check_gap_definition, check_paged_decode, check_e4m3, check_fp8_decode,
        check_paged_fp8_decode, check_decode_attend, check_decode_block_scores,
        check_paged_attend]


@pytest.mark.parametrize("check", PINS, ids=[c.__name__ for c in PINS])
def test_pin(check):
    check(oracle.load())


# --------------------------------------------------------------------------
# 12. Mutation test: plausible mistakes planted in copies of the oracle source
#     (on the CPU) must each fail at least one of the pins above.
# --------------------------------------------------------------------------
MUTANTS = {
    "causal_window_excludes_self": ("if (t_end > i + 1) t_end = i + 1;", "if (t_end > i) t_end = i;"),
    "pool_takes_first_token": ("if (s > best) best = s;", "if (t == b * B) best = s;"),
    "pool_takes_min": ("double best = -INFINITY;", "double best = INFINITY;",
                       "if (s > best) best = s;", "if (s < best) best = s;"),
    "tie_break_larger_id": ("if (best < 0 || S[b] > S[best]) best = b;",
                            "if (best < 0 || S[b] >= S[best]) best = b;"),
    "select_smallest": ("if (best < 0 || S[b] > S[best]) best = b;",
                        "if (best < 0 || S[b] < S[best]) best = b;"),
    "local_not_forced": ("chosen[nchosen++] = (int32_t)bi;         /* local block takes one slot */",
                         "if (bi < 0) chosen[nchosen++] = (int32_t)bi;"),
    "attn_ignores_causal": ("if (t <= i) tok[n++] = t;", "tok[n++] = t;"),
    "wrong_group_of_head": ("int g = h / r;", "int g = h % G;"),
    "scale_dropped": ("z[u] = scale * s;", "z[u] = s;"),
    "values_from_keys": ("const uint16_t *vt = vv + (tok[u] * G + g) * d;",
                         "const uint16_t *vt = kk + (tok[u] * G + g) * d;"),
    "index_key_row_stride": ("const uint16_t *kv = ik + t * dI;", "const uint16_t *kv = ik + t;"),
    "index_group_ignored": ("const uint16_t *qv = iq_row + (int64_t)g * dI;",
                            "const uint16_t *qv = iq_row;"),
    "key_group_ignored": ("const uint16_t *kt = kk + (tok[u] * G + g) * d;",
                          "const uint16_t *kt = kk + (tok[u] * G) * d;"),
    "no_max_subtraction_sign": ("z[u] = exp(z[u] - m);", "z[u] = exp(m - z[u]);"),
    "blocks_after_query_compete": ("int64_t ncand = bi;", "int64_t ncand = bi + 1;"),
    "e4m3_exponent_bias": ("else v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                           "else v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "e4m3_subnormal_scale": ("if (e == 0) v = ldexp((double)m / 8.0, -6);",
                             "if (e == 0) v = ldexp((double)m / 8.0, -7);"),
    "fp8_token_scale_ignored": ("s *= (double)kscale[t];", "s *= 1.0;"),
    "fp8_scale_of_wrong_token": ("s *= (double)kscale[t];", "s *= (double)kscale[b * B];"),
    "decode_key_cache_of_sequence_0": ("const uint16_t *k_n = kc + n * Lmax * G * d;",
                                       "const uint16_t *k_n = kc;"),
    "decode_index_cache_of_sequence_0": ("const uint16_t *ik_n = ikc + n * Lmax * dI;",
                                         "const uint16_t *ik_n = ikc;"),
    "decode_query_one_token_early": ("int64_t i = Ln - 1;", "int64_t i = Ln - 2;"),
    "decode_attend_query_one_token_early": ("int64_t qpos = Ln - 1;", "int64_t qpos = Ln - 2;"),
    "decode_attend_caches_of_sequence_0": ("const uint16_t *kseq = kc + n * Lmax * G * d;",
                                           "const uint16_t *kseq = kc;",
                                           "const uint16_t *vseq = vc + n * Lmax * G * d;",
                                           "const uint16_t *vseq = vc;"),
    "decode_scores_cache_of_sequence_0": ("const uint16_t *iks = ikc + n * Lmax * dI;",
                                          "const uint16_t *iks = ikc;"),
    "decode_scores_fp8_cache_of_sequence_0": ("const uint8_t *ik8s = ik8 + n * Lmax * dI;",
                                              "const uint8_t *ik8s = ik8;"),
    "decode_scores_query_one_token_early": (
        "row_block_scores(iq + n * G * dI, iks, Ln - 1, Ln, G, dI, B, tmp);",
        "row_block_scores(iq + n * G * dI, iks, Ln - 2, Ln, G, dI, B, tmp);"),
    "gap_from_first_pick": ("double a = last, c = S[nxt];", "double a = S[chosen[1]], c = S[nxt];"),
    "gap_not_relative": ("*gap = (den == 0.0) ? 0.0f : (float)(fabs(a - c) / den);",
                         "*gap = (float)fabs(a - c);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle._SRC).read()
    rep = MUTANTS[name]
    for a, b in zip(rep[0::2], rep[1::2]):
        assert src.count(a) >= 1, f"mutation anchor not found: {a}"
        src = src.replace(a, b)
    path = tmp_path / f"{name}.c"
    path.write_text(src)
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", str(so),
                    str(path), "-lm"], check=True)
    lib = oracle.load(str(so))
    caught = []
    for check in PINS:
        try:
            check(lib)
        except AssertionError:
            caught.append(check.__name__)
        except Exception as e:  # a crash of the mutant also counts as caught
            caught.append(f"{check.__name__}:{type(e).__name__}")
    assert caught, f"mutant {name} passed every pin"


def test_torch_e4m3_route_matches_oracle_quantizer():
    """The torch route (frexp + float8_e4m3fn cast) that prepares full-size FP8
    caches on the GPU in the parity tests gives the oracle quantizer's bytes."""
    rng = np.random.default_rng(11)
    x = torch.tensor(rng.standard_normal((3000, 128)) * np.exp(rng.uniform(-30, 30, (3000, 1))),
                     dtype=torch.float32).to(torch.bfloat16)
    x[0] = 0
    c1, s1 = oracle.quantize_e4m3_rows(x)
    c2, s2 = _refs.e4m3_rows_torch(x)
    assert np.array_equal(c1, c2.numpy()) and np.array_equal(s1, s2.numpy())
