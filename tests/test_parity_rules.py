"""CPU checks of the comparison rules the GPU parity tests apply (tests/_parity.py):
the near-tie band check must accept a selection that differs from the oracle's only
among blocks tied at the boundary, and reject one that picks a block below the band
or leaves out a block above it."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import _parity

B, K = 4, 4


def _case():
    """One row, one group, 10 competitors (query in block 10), k - 1 = 3 of them
    selected.  Scores: two clear winners (9, 8) and blocks 1 and 6 tied at the
    boundary (5.0 and 5.0002), everything else at most 4."""
    S = np.full((1, 1, 12), -np.inf, np.float32)
    S[0, 0, :10] = [1, 5.0, 2, 9, 3, 8, 5.0002, 0.5, 0, 4]
    pos = np.array([10 * B + 1])
    ids, gap = oracle.select(S, pos, B, K)
    return S, pos, ids, gap


def test_band_accepts_boundary_swap():
    S, pos, ids, gap = _case()
    assert ids[0, 0].tolist() == [3, 5, 6, 10]          # 9, 8, 5.0002 (+ own block)
    assert gap[0, 0] < _parity.TIE                        # a near-tie row
    swapped = ids.copy()
    swapped[0, 0] = [1, 3, 5, 10]                         # 5.0 instead of 5.0002
    assert _parity.check_near_tie_band(swapped, ids, S, pos, B) == 1
    assert _parity.check_near_tie_band(ids, ids, S, pos, B) == 1


def test_band_rejects_block_below_band():
    S, pos, ids, gap = _case()
    bad = ids.copy()
    bad[0, 0] = [3, 5, 9, 10]                             # 4.0: far below the boundary
    with pytest.raises(AssertionError, match="below the band"):
        _parity.check_near_tie_band(bad, ids, S, pos, B)


def test_band_rejects_missing_winner():
    S, pos, ids, gap = _case()
    bad = ids.copy()
    bad[0, 0] = [1, 5, 6, 10]                             # drops 9.0, takes both tied blocks
    with pytest.raises(AssertionError, match="left out"):
        _parity.check_near_tie_band(bad, ids, S, pos, B)


def test_band_all_competitors_selected():
    """A row whose competitors all fit in the slots has no boundary: the sets must match."""
    S = np.full((1, 1, 4), -np.inf, np.float32)
    S[0, 0, :2] = [1.0, 2.0]
    pos = np.array([2 * B])
    ids, gap = oracle.select(S, pos, B, K)
    assert np.isinf(gap).all()
    assert _parity.check_near_tie_band(ids, ids, S, pos, B) == 0
    bad = ids.copy()
    bad[0, 0, :2] = [1, 1]
    with pytest.raises(AssertionError):
        _parity.check_near_tie_band(bad, ids, S, pos, B)
