"""C-ABI contract tests that need no GPU: the library loads, exports exactly the
symbols include/msa.h declares, sizes its workspaces, and rejects bad arguments
with the documented status codes before launching anything."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_long_idx_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"MSA_API\s+[\w\s\*]+?\b(msa_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(msa.library_path()):
        pytest.skip("libmsa.so not built")
    return msa.load_library()


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("msa_select_blocks", "msa_sparse_attn", "msa_prefill", "msa_prefill_varlen",
                 "msa_decode",
                 "msa_decode_paged", "msa_decode_fp8idx", "msa_decode_paged_fp8idx",
                 "msa_quantize_idx_k_e4m3",
                 "msa_select_blocks_workspace_size",
                 "msa_sparse_attn_workspace_size", "msa_prefill_workspace_size",
                 "msa_decode_workspace_size", "msa_decode_paged_workspace_size",
                 "msa_status_string"):
        assert want in names


def test_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", msa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)
    # nothing beyond the declared C ABI is exported as a function
    assert {n for n in exported if n.startswith("msa")} == set(_declared())


def test_status_strings(lib):
    assert lib.msa_status_string(0) == b"MSA_OK"
    assert lib.msa_status_string(3) == b"MSA_ERR_WORKSPACE_TOO_SMALL"
    assert lib.msa_status_string(99) == b"MSA_ERR_UNKNOWN"


def test_workspace_sizes(lib):
    assert lib.msa_select_blocks_workspace_size(0, 4, 128, 128, 16) == 0
    s1 = lib.msa_select_blocks_workspace_size(4096, 2, 32, 128, 4)
    assert s1 >= 4096 * 2 * 32 * 4
    s2 = lib.msa_prefill_workspace_size(131072, 64, 4, 128, 128, 128, 16)
    # bounded by the query chunk, not by L
    s3 = lib.msa_prefill_workspace_size(1048576, 64, 4, 128, 128, 128, 16)
    assert s2 > 0 and s3 < 4 * s2 + (1 << 34)
    assert lib.msa_decode_workspace_size(64, 262144, 64, 4, 128, 128, 128, 16) > 0
    # paged decode: the contiguous decode workspace at Lmax = max_blocks * B, plus one
    # checked length per sequence
    wp = lib.msa_decode_paged_workspace_size(64, 2048, 64, 4, 128, 128, 128, 16)
    assert wp >= lib.msa_decode_workspace_size(64, 262144, 64, 4, 128, 128, 128, 16) + 64 * 4
    assert lib.msa_decode_paged_workspace_size(0, 2048, 64, 4, 128, 128, 128, 16) == 0


P = ctypes.c_void_p


def _fake(n=1 << 20):
    """A host address used only as a non-null token: every call below must fail
    validation before it could be dereferenced."""
    return P(0x1000)


def test_invalid_and_unsupported_arguments(lib):
    f = _fake()
    ws = P(0x100000)   # 256-byte aligned token
    big = ctypes.c_size_t(1 << 40)
    s = None
    # null pointers with L > 0
    assert lib.msa_select_blocks(None, f, 256, 2, 32, 128, 4, f, ws, big, s) == INVALID
    # k < 1, negative L
    assert lib.msa_select_blocks(f, f, 256, 2, 32, 128, 0, f, ws, big, s) == INVALID
    assert lib.msa_select_blocks(f, f, -1, 2, 32, 128, 4, f, ws, big, s) == INVALID
    # unsupported: B != 128, dI, k > 32, G*dI > 512
    assert lib.msa_select_blocks(f, f, 256, 2, 32, 64, 4, f, ws, big, s) == UNSUPPORTED
    assert lib.msa_select_blocks(f, f, 256, 2, 48, 128, 4, f, ws, big, s) == UNSUPPORTED
    assert lib.msa_select_blocks(f, f, 256, 2, 32, 128, 33, f, ws, big, s) == UNSUPPORTED
    assert lib.msa_select_blocks(f, f, 256, 8, 128, 128, 4, f, ws, big, s) == UNSUPPORTED
    # workspace too small / misaligned
    assert lib.msa_select_blocks(f, f, 256, 2, 32, 128, 4, f, ws, ctypes.c_size_t(16), s) == WS_SMALL
    assert lib.msa_select_blocks(f, f, 256, 2, 32, 128, 4, f, P(0x100010), big, s) == WS_SMALL
    # sparse attention: H % G, d, r
    assert lib.msa_sparse_attn(f, f, f, f, 256, 6, 4, 64, 128, 4, ctypes.c_float(0), f, ws, big,
                               s) == INVALID
    assert lib.msa_sparse_attn(f, f, f, f, 256, 8, 2, 96, 128, 4, ctypes.c_float(0), f, ws, big,
                               s) == UNSUPPORTED
    assert lib.msa_sparse_attn(f, f, f, f, 256, 128, 2, 64, 128, 4, ctypes.c_float(0), f, ws, big,
                               s) == UNSUPPORTED
    # prefill and decode null / size checks
    assert lib.msa_prefill(f, f, f, f, None, 256, 8, 2, 64, 32, 128, 4, ctypes.c_float(0), f, None,
                           ws, big, s) == INVALID
    assert lib.msa_decode(f, f, f, f, f, None, 2, 1024, 8, 2, 64, 32, 128, 4, ctypes.c_float(0), f,
                          None, ws, big, s) == INVALID
    assert lib.msa_decode(f, f, f, f, f, f, 2, 1024, 8, 2, 64, 32, 128, 4, ctypes.c_float(0), f,
                          None, ws, ctypes.c_size_t(8), s) == WS_SMALL


def test_empty_inputs_are_no_ops(lib):
    # L == 0 / N == 0: valid empty problems, nothing launched, null pointers allowed
    assert lib.msa_select_blocks(None, None, 0, 2, 32, 128, 4, None, None, 0, None) == OK
    assert lib.msa_sparse_attn(None, None, None, None, 0, 8, 2, 64, 128, 4, ctypes.c_float(0),
                               None, None, 0, None) == OK
    assert lib.msa_prefill(None, None, None, None, None, 0, 8, 2, 64, 32, 128, 4,
                           ctypes.c_float(0), None, None, None, 0, None) == OK
    assert lib.msa_decode(None, None, None, None, None, None, 0, 1024, 8, 2, 64, 32, 128, 4,
                          ctypes.c_float(0), None, None, None, 0, None) == OK


def test_binding_fails_loudly_without_gpu_tensors():
    import torch
    if not os.path.exists(msa.library_path()):
        pytest.skip("libmsa.so not built")
    x = torch.zeros(4, 2, 32, dtype=torch.bfloat16)
    with pytest.raises(msa.MSAError):
        msa.select_blocks(x, torch.zeros(4, 32, dtype=torch.bfloat16), k=4)


def test_paged_decode_arguments(lib):
    f, ws, big, s = _fake(), P(0x100000), ctypes.c_size_t(1 << 40), None
    zero = ctypes.c_float(0)

    def call(q=f, table=f, seq_len=f, N=2, npages=16, maxb=8, H=8, G=2, d=64, dI=32, B=128, k=4,
             ws_=ws, nbytes=big):
        return lib.msa_decode_paged(q, f, f, f, f, npages, table, maxb, seq_len, N, H, G, d, dI, B,
                                    k, zero, f, None, ws_, nbytes, s)

    assert call(N=0, q=None, table=None, seq_len=None) == OK      # empty batch: nothing to do
    assert call(table=None) == INVALID
    assert call(seq_len=None) == INVALID
    assert call(npages=0) == INVALID
    assert call(maxb=0) == INVALID
    assert call(H=6, G=4) == INVALID
    assert call(B=64) == UNSUPPORTED        # a page is one 128-token MSA block
    assert call(d=96) == UNSUPPORTED
    assert call(k=33) == UNSUPPORTED
    assert call(maxb=1 << 24) == UNSUPPORTED  # max_blocks * 128 must fit in int32
    assert call(nbytes=ctypes.c_size_t(64)) == WS_SMALL
    assert call(ws_=P(0x100010)) == WS_SMALL


def test_fp8_decode_and_quantizer_arguments(lib):
    f, ws, big, s = _fake(), P(0x100000), ctypes.c_size_t(1 << 40), None
    zero = ctypes.c_float(0)

    def call(q=f, ik8=f, sc=f, N=2, Lmax=1024, H=8, G=2, d=64, dI=32, B=128, k=4, nbytes=big):
        return lib.msa_decode_fp8idx(q, f, f, f, ik8, sc, f, N, Lmax, H, G, d, dI, B, k, zero, f,
                                     None, ws, nbytes, s)

    assert call(N=0, q=None, ik8=None, sc=None) == OK
    assert call(ik8=None) == INVALID
    assert call(sc=None) == INVALID
    assert call(Lmax=0) == INVALID
    assert call(B=64) == UNSUPPORTED
    assert call(dI=48) == UNSUPPORTED
    assert call(nbytes=ctypes.c_size_t(16)) == WS_SMALL
    # cache writer
    assert lib.msa_quantize_idx_k_e4m3(None, 0, 128, None, None, s) == OK
    assert lib.msa_quantize_idx_k_e4m3(None, 10, 128, f, f, s) == INVALID
    assert lib.msa_quantize_idx_k_e4m3(f, 10, 128, f, None, s) == INVALID
    assert lib.msa_quantize_idx_k_e4m3(f, -1, 128, f, f, s) == INVALID
    assert lib.msa_quantize_idx_k_e4m3(f, 10, 96, f, f, s) == UNSUPPORTED


def test_varlen_prefill_arguments(lib):
    f, ws, big, s = _fake(), P(0x100000), ctypes.c_size_t(1 << 40), None
    zero = ctypes.c_float(0)
    I64 = ctypes.c_int64

    def call(cu_q, cu_kv, nseq=None, q=f, H=8, G=2, d=64, dI=32, B=128, k=4, nbytes=big):
        n = len(cu_q) - 1 if nseq is None else nseq
        aq = (I64 * len(cu_q))(*cu_q) if cu_q is not None else None
        akv = (I64 * len(cu_kv))(*cu_kv) if cu_kv is not None else None
        return lib.msa_prefill_varlen(q, f, f, f, f, aq, akv, n, H, G, d, dI, B, k, zero, f, None,
                                      ws, nbytes, s)

    assert call(None, None, nseq=0) == OK
    assert call([0, 0, 0], [0, 300, 600], q=None) == OK        # no new tokens: nothing to do
    assert call(None, [0, 10], nseq=1) == INVALID
    assert call([0, 300], [0, 200]) == INVALID                 # more new tokens than tokens
    assert call([0, 10, 5], [0, 10, 20]) == INVALID            # decreasing offsets
    assert call([0, 100], [0, 200]) == UNSUPPORTED             # prefix of 100: not whole blocks
    assert call([0, 100], [0, 1048576 + 228]) == UNSUPPORTED   # longer than 2^20 tokens
    assert call([0, 100], [0, 100], B=64) == UNSUPPORTED
    assert call([0, 100], [0, 100], nbytes=ctypes.c_size_t(64)) == WS_SMALL


def test_varlen_workspace_size(lib):
    """The varlen workspace size is host arithmetic: the single-sequence size for one
    sequence, and the size of the largest batch (at most 128 sequences) otherwise."""
    I64 = ctypes.c_int64

    def ws(cu_q, cu_kv, H=16, G=4, d=128, dI=128, k=8):
        aq, akv = (I64 * len(cu_q))(*cu_q), (I64 * len(cu_kv))(*cu_kv)
        return lib.msa_prefill_varlen_workspace_size(aq, akv, len(cu_q) - 1, H, G, d, dI, 128, k)

    def single(L, k=8):
        return lib.msa_prefill_workspace_size(L, 16, 4, 128, 128, 128, k)

    assert lib.msa_prefill_varlen_workspace_size(None, None, 0, 16, 4, 128, 128, 128, 8) == 0
    assert ws([0, 5000], [0, 5000]) == single(5000)
    # sequences of more than k blocks (640 tokens, k = 4) are batched
    cu = [640 * i for i in range(65)]              # 64 sequences, one batch
    assert ws(cu, cu, k=4) > single(640, k=4)
    assert ws(cu, cu, k=4) >= 64 * 640 * 16 * 4 * 128 * 2   # the partials of every row
    cu2 = [640 * i for i in range(201)]            # 200 sequences: batches of 128 and 72
    assert ws(cu2, cu2, k=4) == ws(cu2[:129], cu2[:129], k=4)
    # sequences of at most k blocks run the dense main branch, which needs no batch
    # workspace: only the single-sequence size remains
    cu3 = [512 * i for i in range(65)]
    assert ws(cu3, cu3) == single(512)
    # a sequence with nothing new adds nothing
    assert ws([0, 0, 300], [0, 4096, 4396]) == ws([0, 300], [0, 300])
    # more than 8192 new tokens: that sequence runs alone, with its own workspace size
    assert ws([0, 20000, 20500, 21000], [0, 20000, 20500, 21000]) == single(20000)


def test_paged_fp8_decode_arguments(lib):
    f, ws, big, s = _fake(), P(0x100000), ctypes.c_size_t(1 << 40), None
    zero = ctypes.c_float(0)

    def call(ik8=f, sc=f, table=f, N=2, npages=16, maxb=8, B=128, dI=32, nbytes=big):
        return lib.msa_decode_paged_fp8idx(f, f, f, f, ik8, sc, npages, table, maxb, f, N, 8, 2,
                                           64, dI, B, 4, zero, f, None, ws, nbytes, s)

    assert call(N=0, ik8=None, sc=None, table=None) == OK
    assert call(ik8=None) == INVALID
    assert call(sc=None) == INVALID
    assert call(table=None) == INVALID
    assert call(npages=0) == INVALID
    assert call(B=64) == UNSUPPORTED
    assert call(dI=48) == UNSUPPORTED
    assert call(nbytes=ctypes.c_size_t(64)) == WS_SMALL


def test_decode_static_refuses_oversize_before_any_launch(lib):
    """msa_decode_static (the decode for callers that cannot allocate) refuses a shape
    whose workspace exceeds its per-GPU array, before any HIP call -- so this runs
    without a GPU and never dereferences the (dummy) pointers."""
    N, Lmax, H, G, d, dI, k = 64, 1 << 24, 64, 4, 128, 128, 16
    assert lib.msa_decode_workspace_size(N, Lmax, H, G, d, dI, 128, k) > msa.STATIC_SCRATCH_BYTES
    dummy = ctypes.c_void_p(256)
    assert lib.msa_decode_static(dummy, dummy, dummy, dummy, dummy, dummy, N, Lmax, H, G, d, dI,
                                 128, k, 0.0, dummy, None, None) == WS_SMALL
    assert lib.msa_decode_static(None, dummy, dummy, dummy, dummy, dummy, 4, 1024, H, G, d, dI,
                                 128, k, 0.0, dummy, None, None) == INVALID
    src = open(HEADER).read()
    assert "#define MSA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)" in src
    assert msa.STATIC_SCRATCH_BYTES == 64 << 20
