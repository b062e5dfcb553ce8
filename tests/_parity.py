"""Comparison rules between the HIP path and the oracle (test helpers).

Block ids: bit-exact on every (query, group) row whose boundary gap (relative
difference between the last selected and the first unselected competitor score,
taken on the oracle's fp32 block scores) is at least 1e-4; rows below that are
near-ties -- reported, not counted, but still checked for validity.
Outputs: bf16 results within max-abs 2e-2 and mean-abs 2e-3 of the oracle's fp64
attention.  On near-tie rows the GPU's own (valid) selection is attended by the
oracle and compared instead.
"""
from __future__ import annotations

import numpy as np

import oracle

TIE = 1e-4
MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def check_selection_valid(ids: np.ndarray, pos: np.ndarray, k: int, B: int = 128):
    """Invariants of a selection: own block present, ids unique, ascending, in
    [0, b(i)], count min(k, b(i)+1), -1 padding at the end."""
    bi = pos // B
    n = np.minimum(k, bi + 1)
    slot = np.arange(k)[None, None, :]
    valid = slot < n[:, None, None]
    assert np.all(np.where(valid, ids >= 0, ids == -1)), "padding/validity"
    assert np.all(np.where(valid, ids <= bi[:, None, None], True)), "id beyond own block"
    d = np.diff(ids, axis=-1)
    vnext = valid[..., 1:]
    assert np.all(np.where(vnext, d > 0, True)), "not strictly ascending"
    last = np.take_along_axis(ids, (n - 1)[:, None, None].repeat(ids.shape[1], 1), axis=-1)[..., 0]
    assert np.all(last == bi[:, None]), "own block missing"


def compare_ids(gpu_ids: np.ndarray, ora_ids: np.ndarray, gap: np.ndarray):
    """Returns (near_tie_mask [n,G], n_mismatch_outside_ties)."""
    tie = gap < TIE
    mism = np.any(gpu_ids != ora_ids, axis=-1) & ~tie
    return tie, int(mism.sum())


def check_near_tie_band(gpu_ids: np.ndarray, ora_ids: np.ndarray, S: np.ndarray,
                        pos: np.ndarray, B: int = 128) -> int:
    """On near-tie rows the GPU may pick other competitors than the oracle, but only
    inside the tie band.  gpu_ids / ora_ids [n, G, k] and the oracle's fp32 block
    scores S [n, G, >= b(i)] of the same n rows (query positions pos).  With
    a = the lowest score the oracle selected among the competitors (blocks < b(i)),
    c = the highest score it left out, and the band delta = 1e-4 * max(|a|, |c|):
      - every competitor the GPU selected scores at least a - delta, and
      - every competitor scoring above c + delta is selected by the GPU,
    so the two selections can differ only among blocks within the band around the
    boundary.  Returns the number of (row, group) pairs checked."""
    n, G, _ = gpu_ids.shape
    checked = 0
    for r in range(n):
        bi = int(pos[r]) // B
        for g in range(G):
            sv = S[r, g, :bi].astype(np.float64)
            oc = [int(b) for b in ora_ids[r, g] if 0 <= b < bi]
            gc = [int(b) for b in gpu_ids[r, g] if 0 <= b < bi]
            if len(oc) == bi:          # every competitor selected: no boundary
                assert sorted(gc) == sorted(oc), (r, g, gc, oc)
                continue
            left = np.ones(bi, bool)
            left[oc] = False
            a = sv[oc].min() if oc else np.inf
            c = sv[left].max()
            delta = TIE * max(abs(a), abs(c)) if np.isfinite(a) else 0.0
            assert len(gc) == len(oc), (r, g, gc, oc)
            low = [b for b in gc if sv[b] < a - delta]
            assert not low, f"row {r} group {g}: GPU picked {low} below the band ({a}, {c})"
            must = np.nonzero(sv > c + delta)[0]
            miss = sorted(set(must.tolist()) - set(gc))
            assert not miss, f"row {r} group {g}: GPU left out {miss} above the band ({a}, {c})"
            checked += 1
    return checked


def compare_out(gpu_out: np.ndarray, ref: np.ndarray):
    err = np.abs(gpu_out.astype(np.float64) - ref)
    return float(err.max()), float(err.mean())


def prefill_rows_vs_oracle(x: dict, rows: np.ndarray, gpu_ids: np.ndarray, gpu_out: np.ndarray,
                           B: int, k: int, scale: float):
    """Oracle on the given rows; returns a dict of parity statistics.  gpu_ids /
    gpu_out are the GPU results of those rows (numpy)."""
    ids, gap, out = oracle.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], B, k, scale, rows=rows)
    check_selection_valid(gpu_ids, rows, k, B)
    tie, nmis = compare_ids(gpu_ids, ids, gap)
    ref = out.copy()
    banded = 0
    if tie.any():
        tie_rows = np.nonzero(tie.any(axis=1))[0]
        # the GPU's competitors on near-tie rows lie inside the tie band
        S = oracle.block_scores(x["iq"], x["ik"], B, rows=rows[tie_rows])
        banded = check_near_tie_band(gpu_ids[tie_rows], ids[tie_rows], S, rows[tie_rows], B)
        # attend the GPU's own selection on near-tie rows
        alt = oracle.attend(x["q"], x["k"], x["v"], gpu_ids[tie_rows], B, scale,
                            rows=rows[tie_rows])
        ref[tie_rows] = alt
    mx, mean = compare_out(gpu_out, ref)
    return {"rows": len(rows), "near_ties": int(tie.sum()), "band_checked": banded,
            "id_mismatches": nmis, "max_abs": mx, "mean_abs": mean}
