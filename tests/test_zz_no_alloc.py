"""msa_decode_static -- decode with the library's own per-GPU workspace array, for
callers that cannot allocate device memory -- against msa_decode with a caller
workspace: the same kernels, so ids and outputs must be bitwise equal, on two calls
in a row (the second smaller, so it runs over the first call's leftovers in the
array), and a shape whose workspace exceeds the array is refused."""
from __future__ import annotations

import ctypes
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import _parity

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[no-alloc] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_idx_amd as msa
    msa.load_library()
    yield
    torch.cuda.synchronize()


def _case(shape, seq_len, seed):
    import block_sparse_long_idx_amd as msa
    x = synth.decode_inputs(shape, seed=seed, seq_len=np.clip(seq_len, 1, shape.Lc))
    d = {n: x[n].to(DEV) for n in ("q", "iq", "k_cache", "v_cache", "ik_cache")}
    sl = torch.tensor(np.asarray(seq_len, np.int32), device=DEV)
    need = msa.workspace_size("decode", N=shape.N, Lmax=shape.Lc, H=shape.H, G=shape.G, d=shape.d,
                              dI=shape.dI, k=shape.k)
    assert need <= msa.STATIC_SCRATCH_BYTES
    o_ref, i_ref = msa.decode(d["q"], d["iq"], d["k_cache"], d["v_cache"], d["ik_cache"], sl,
                              kslots=shape.k, return_ids=True)
    out = torch.empty_like(d["q"])
    ids = torch.empty((shape.N, shape.G, shape.k), dtype=torch.int32, device=DEV)
    msa.decode_static(d["q"], d["iq"], d["k_cache"], d["v_cache"], d["ik_cache"], sl,
                      kslots=shape.k, return_ids=True, out=out, ids_out=ids)
    torch.cuda.synchronize()
    return x, o_ref, i_ref, out, ids


def test_decode_static_matches_decode_twice():
    # first call: 8 sequences x 12000 tokens, k = 32 (the split attention form, whose
    # partials use the array too); second: 3 sequences x 1500 tokens, k = 16
    big = synth.DecodeShape(N=8, Lc=12000, H=64, G=4, d=128, dI=128, B=128, k=32)
    small = synth.DecodeShape(N=3, Lc=1500, H=64, G=4, d=128, dI=128, B=128, k=16)
    for shape, seq_len, seed in ((big, [12000, 9000, 4097, 129, 1, 0, 11111, 12001], 5),
                                 (small, [1500, 700, 129], 6)):
        _say(f"N={shape.N} Lmax={shape.Lc} k={shape.k} seq_len={seq_len}")
        x, o_ref, i_ref, out, ids = _case(shape, seq_len, seed)
        assert torch.equal(ids, i_ref)
        assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16))
        # and the oracle on the valid sequences
        lens = np.asarray(seq_len)
        valid = np.nonzero((lens >= 1) & (lens <= shape.Lc))[0]
        scale = 1.0 / math.sqrt(shape.d)
        oids, gap, oout = oracle.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"],
                                        x["ik_cache"], np.clip(lens, 1, shape.Lc), 128, shape.k,
                                        scale, seqs=valid)
        tie, nmis = _parity.compare_ids(ids.cpu().numpy()[valid], oids, gap)
        assert nmis == 0
        keep = ~tie.any(axis=1)
        mx, mean = _parity.compare_out(out.float().cpu().numpy()[valid][keep], oout[keep])
        _say(f"  -> bitwise equal to msa_decode; oracle max {mx:.3e} mean {mean:.3e}")
        assert mx < _parity.MAX_ABS and mean < _parity.MEAN_ABS


def test_decode_static_refuses_a_shape_beyond_the_array():
    import block_sparse_long_idx_amd as msa
    lib = msa.load_library()
    N, Lmax, H, G, d, dI, k = 64, 1 << 24, 64, 4, 128, 128, 16
    assert lib.msa_decode_workspace_size(N, Lmax, H, G, d, dI, 128, k) > msa.STATIC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)        # never dereferenced: the size check comes first
    st = lib.msa_decode_static(dummy, dummy, dummy, dummy, dummy, dummy, N, Lmax, H, G, d, dI,
                               128, k, 0.0, dummy, None, None)
    assert st == 3                      # MSA_ERR_WORKSPACE_TOO_SMALL
