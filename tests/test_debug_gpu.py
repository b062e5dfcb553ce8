"""The MSA_DEBUG_SYNC=1 debug mode (every kernel stage followed by a synchronisation
that reports a fault at the stage that caused it; the library reads the variable at
every stage) changes no result: prefill and decode give bitwise the same ids and
outputs with it on and off."""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run():
    import block_sparse_long_idx_amd as msa
    sh = synth.PrefillShape(L=3000, H=16, G=4, d=128, dI=128, B=128, k=8)
    x = synth.prefill_inputs(sh, seed=2)
    o, i = msa.prefill(*(x[n].to(DEV) for n in ("q", "k", "v", "iq", "ik")), kslots=sh.k,
                       return_ids=True)
    ds = synth.DecodeShape(N=4, Lc=2000, H=16, G=4, d=128, dI=128, B=128, k=8)
    y = synth.decode_inputs(ds, seed=3, seq_len=[2000, 999, 129, 1])
    sl = torch.tensor([2000, 999, 129, 1], dtype=torch.int32, device=DEV)
    do, di = msa.decode(*(y[n].to(DEV) for n in ("q", "iq", "k_cache", "v_cache", "ik_cache")),
                        sl, kslots=ds.k, return_ids=True)
    torch.cuda.synchronize()
    return [t.cpu() for t in (o.view(torch.int16), i, do.view(torch.int16), di)]


def test_debug_sync_changes_no_result():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    old = os.environ.get("MSA_DEBUG_SYNC")
    try:
        os.environ["MSA_DEBUG_SYNC"] = "0"
        plain = _run()
        os.environ["MSA_DEBUG_SYNC"] = "1"
        debug = _run()
    finally:
        if old is None:
            os.environ.pop("MSA_DEBUG_SYNC", None)
        else:
            os.environ["MSA_DEBUG_SYNC"] = old
    for a, b in zip(plain, debug):
        assert torch.equal(a, b)
