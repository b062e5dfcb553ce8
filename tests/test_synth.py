"""Input generators that need no GPU: the constructed skewed block ids satisfy the
contract of msa_sparse_attn's block_ids and make the chosen blocks hot."""
from __future__ import annotations

import numpy as np
import torch

import synth


def test_skewed_ids_structure():
    L, G, k, hot = 5000, 3, 16, (0, 1, 2, 3)
    ids = synth.skewed_ids(L, G, k, hot=hot, seed=7).numpy()
    assert ids.shape == (L, G, k) and ids.dtype == np.int32
    bi = np.arange(L) // 128
    for i in range(L):
        for g in range(G):
            row = ids[i, g]
            if bi[i] < k:
                # every block of the causal window, then padding
                n = bi[i] + 1
                assert (row[:n] == np.arange(n)).all() and (row[n:] == -1).all()
            else:
                assert (np.diff(row) > 0).all()                   # ascending, unique
                assert row[-1] == bi[i]                            # own block present
                assert (row[:len(hot)] == np.arange(len(hot))).all()  # hot blocks present
                assert row.min() >= 0


def test_skewed_ids_seeded_and_spread():
    a = synth.skewed_ids(4096, 2, 8, seed=1)
    assert torch.equal(a, synth.skewed_ids(4096, 2, 8, seed=1))
    assert not torch.equal(a, synth.skewed_ids(4096, 2, 8, seed=2))
    # the drawn blocks of late rows cover the non-hot range roughly uniformly
    late = a[3072:, :, 4:7].numpy().ravel()
    hist = np.bincount(late, minlength=32)[4:24]
    assert hist.min() > 0.5 * hist.mean()
