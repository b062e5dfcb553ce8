"""CPU oracle for the MSA forward pass -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its binding) never
does.  The arithmetic lives in ``msa_oracle.c`` (plain C, fp64 accumulation,
OpenMP over query rows); this module only compiles it with gcc and marshals
numpy arrays into it.  See the header of ``msa_oracle.c`` for the passages each
step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (-O2, OpenMP).  Always recompiles."""
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: str | None = None):
    """Load the compiled oracle; compile it first only if nothing is built."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_block_scores.argtypes = [P, P, i64, i32, i32, i32, P, i64, P]
    lib.oracle_select.argtypes = [P, P, i64, i32, i64, i32, i32, P, P]
    lib.oracle_attend.argtypes = [P, P, P, P, P, i64, i64, i32, i32, i32, i32, i32, f64, P]
    lib.oracle_prefill_rows.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, f64,
                                        P, i64, P, P, P]
    lib.oracle_decode.argtypes = [P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, f64,
                                  P, i64, P, P, P]
    lib.oracle_decode_attend.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, f64, P, i64,
                                         P, P]
    lib.oracle_decode_block_scores.argtypes = [P, P, P, i64, i32, i32, i32, P, i64, i64, P]
    lib.oracle_decode_block_scores_fp8.argtypes = [P, P, P, P, i64, i32, i32, i32, P, i64, i64,
                                                   P]
    lib.oracle_e4m3_table.argtypes = [P]
    lib.oracle_decode_fp8idx.argtypes = [P, P, P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32,
                                         f64, P, i64, P, P, P]
    for f in (lib.oracle_block_scores, lib.oracle_select, lib.oracle_attend,
              lib.oracle_prefill_rows, lib.oracle_decode, lib.oracle_decode_attend,
              lib.oracle_e4m3_table, lib.oracle_decode_fp8idx, lib.oracle_decode_block_scores,
              lib.oracle_decode_block_scores_fp8):
        f.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    if path is None:
        _lib = lib
    return lib


def num_threads(lib=None) -> int:
    return int((lib or load()).oracle_num_threads())


def _u16(a) -> np.ndarray:
    """bf16 data as a contiguous uint16 numpy array (torch bf16 tensors accepted)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    except ImportError:  # pragma: no cover - torch is always present in this image
        pass
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows, L):
    if rows is None:
        rows = np.arange(L, dtype=np.int64)
    return np.ascontiguousarray(np.asarray(rows, dtype=np.int64))


def block_scores(iq, ik, B, rows=None, lib=None):
    """S[nrows, G, nb] fp32; entries outside the causal window are -inf."""
    lib = lib or load()
    iq, ik = _u16(iq), _u16(ik)
    L, G, dI = iq.shape
    rows = _rows(rows, L)
    nb = (L + B - 1) // B
    S = np.empty((len(rows), G, nb), np.float32)
    lib.oracle_block_scores(_ptr(iq), _ptr(ik), L, G, dI, B, _ptr(rows), len(rows), _ptr(S))
    return S


def select(S, rows, B, k, lib=None):
    """ids[nrows, G, k] (ascending, -1 padded) and gap[nrows, G] from block scores."""
    lib = lib or load()
    S = np.ascontiguousarray(S, dtype=np.float32)
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    n, G, nb = S.shape
    ids = np.empty((n, G, k), np.int32)
    gap = np.empty((n, G), np.float32)
    lib.oracle_select(_ptr(S), _ptr(rows), n, G, nb, B, k, _ptr(ids), _ptr(gap))
    return ids, gap


def attend(q, k, v, ids, B, scale, rows=None, lib=None):
    """out[nrows, H, d] float64: exact softmax attention over the given blocks."""
    lib = lib or load()
    q, kk, vv = _u16(q), _u16(k), _u16(v)
    L, H, d = q.shape
    G = kk.shape[1]
    rows = _rows(rows, L)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    kslots = ids.shape[2]
    out = np.empty((len(rows), H, d), np.float64)
    lib.oracle_attend(_ptr(q), _ptr(kk), _ptr(vv), _ptr(ids), _ptr(rows), len(rows), L, H, G, d,
                      B, kslots, float(scale), _ptr(out))
    return out


def prefill(q, k, v, iq, ik, B, kslots, scale=None, rows=None, lib=None):
    """Full MSA prefill for the listed rows: (ids, gap, out)."""
    lib = lib or load()
    q, kk, vv, iq, ik = _u16(q), _u16(k), _u16(v), _u16(iq), _u16(ik)
    L, H, d = q.shape
    G, dI = iq.shape[1], iq.shape[2]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = _rows(rows, L)
    n = len(rows)
    ids = np.empty((n, G, kslots), np.int32)
    gap = np.empty((n, G), np.float32)
    out = np.empty((n, H, d), np.float64)
    lib.oracle_prefill_rows(_ptr(q), _ptr(kk), _ptr(vv), _ptr(iq), _ptr(ik), L, H, G, d, dI, B,
                            kslots, float(scale), _ptr(rows), n, _ptr(ids), _ptr(gap), _ptr(out))
    return ids, gap, out


def decode(q, iq, k_cache, v_cache, ik_cache, seq_len, B, kslots, scale=None, seqs=None,
           lib=None):
    """MSA decode (query = last cached token of each sequence): (ids, gap, out)."""
    lib = lib or load()
    q, iq = _u16(q), _u16(iq)
    kc, vc, ikc = _u16(k_cache), _u16(v_cache), _u16(ik_cache)
    N, H, d = q.shape
    G, dI = iq.shape[1], iq.shape[2]
    Lmax = kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    seq_len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64))
    seqs = _rows(seqs, N)
    n = len(seqs)
    ids = np.empty((n, G, kslots), np.int32)
    gap = np.empty((n, G), np.float32)
    out = np.empty((n, H, d), np.float64)
    lib.oracle_decode(_ptr(q), _ptr(iq), _ptr(kc), _ptr(vc), _ptr(ikc), _ptr(seq_len), Lmax, H,
                      G, d, dI, B, kslots, float(scale), _ptr(seqs), n, _ptr(ids), _ptr(gap),
                      _ptr(out))
    return ids, gap, out


def decode_attend(q, k_cache, v_cache, seq_len, ids, B, scale, seqs, lib=None):
    """Decode main branch for the listed sequences with given ids [nseqs, G, k]."""
    lib = lib or load()
    q, kc, vc = _u16(q), _u16(k_cache), _u16(v_cache)
    N, H, d = q.shape
    Lmax, G = kc.shape[1], kc.shape[2]
    seq_len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64))
    seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    out = np.empty((len(seqs), H, d), np.float64)
    lib.oracle_decode_attend(_ptr(q), _ptr(kc), _ptr(vc), _ptr(seq_len), Lmax, H, G, d, B,
                             ids.shape[2], float(scale), _ptr(seqs), len(seqs), _ptr(ids),
                             _ptr(out))
    return out


def decode_block_scores(iq, ik_cache, seq_len, B, seqs, lib=None):
    """Decode block scores S[nseqs, G, nbmax] (fp32) of the listed sequences: the
    query at position seq_len[n]-1 against sequence n's own index keys; blocks past
    the query's own block are -inf.  nbmax = ceil(max listed seq_len / B)."""
    lib = lib or load()
    iq, ikc = _u16(iq), _u16(ik_cache)
    N, G, dI = iq.shape
    Lmax = ikc.shape[1]
    seq_len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64))
    seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    nbmax = int((seq_len[seqs].max() + B - 1) // B) if len(seqs) else 1
    S = np.empty((len(seqs), G, nbmax), np.float32)
    lib.oracle_decode_block_scores(_ptr(iq), _ptr(ikc), _ptr(seq_len), Lmax, G, dI, B,
                                   _ptr(seqs), len(seqs), nbmax, _ptr(S))
    return S


def decode_block_scores_fp8(iq, ik8, kscale, seq_len, B, seqs, lib=None):
    """As decode_block_scores, over an E4M3 index-key cache with per-token scales."""
    lib = lib or load()
    iq = _u16(iq)
    ik8 = np.ascontiguousarray(ik8.cpu().numpy() if hasattr(ik8, "cpu") else ik8, np.uint8)
    ks = np.ascontiguousarray(kscale.cpu().numpy() if hasattr(kscale, "cpu") else kscale,
                              np.float32)
    N, G, dI = iq.shape
    Lmax = ik8.shape[1]
    seq_len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64))
    seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    nbmax = int((seq_len[seqs].max() + B - 1) // B) if len(seqs) else 1
    S = np.empty((len(seqs), G, nbmax), np.float32)
    lib.oracle_decode_block_scores_fp8(_ptr(iq), _ptr(ik8), _ptr(ks), _ptr(seq_len), Lmax, G, dI,
                                       B, _ptr(seqs), len(seqs), nbmax, _ptr(S))
    return S


def decode_paged_block_scores(iq, ik_pages, block_table, seq_len, B, seqs, lib=None):
    """Decode block scores of the listed (valid) sequences of a paged cache: the
    sequence's index-key pages gathered in logical order, then decode_block_scores."""
    iq, ikp = _u16(iq), _u16(ik_pages)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                       dtype=np.int64)
    lens = np.asarray(seq_len.cpu() if hasattr(seq_len, "cpu") else seq_len, dtype=np.int64)
    dI = ikp.shape[2]
    seqs = np.asarray(seqs, np.int64)
    nbmax = int((lens[seqs].max() + B - 1) // B) if len(seqs) else 1
    S = np.full((len(seqs), iq.shape[1], nbmax), -np.inf, np.float32)
    for r, n in enumerate(seqs):
        pages = _pages_of(table, lens, n, B, ikp.shape[0])
        if pages is None:
            raise ValueError(f"sequence {n} is not valid")
        Lc = len(pages) * B
        s1 = decode_block_scores(iq[n:n + 1], ikp[pages].reshape(1, Lc, dI), [int(lens[n])], B,
                                 [0], lib=lib)
        S[r, :, :s1.shape[2]] = s1[0]
    return S


def decode_paged(q, iq, k_pages, v_pages, ik_pages, block_table, seq_len, B, kslots, scale=None,
                 seqs=None, lib=None):
    """Paged MSA decode for the listed sequences: (ids, gap, out, valid).

    Token t of sequence n is row t % B of page block_table[n, t // B] (every MSA block
    is one cache page).  The listed sequences' pages are gathered, in logical
    order, into contiguous caches, and the contiguous decode above runs on them.  A
    sequence whose length is outside [1, max_blocks * B] or that needs a page id
    outside [0, num_pages) is not computed: valid False, ids -1, out 0, gap nan.
    """
    q, iq = _u16(q), _u16(iq)
    kp, vp, ikp = _u16(k_pages), _u16(v_pages), _u16(ik_pages)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                       dtype=np.int64)
    lens = np.asarray(seq_len.cpu() if hasattr(seq_len, "cpu") else seq_len, dtype=np.int64)
    N, H, d = q.shape
    G, dI = iq.shape[1], iq.shape[2]
    npages, maxb = kp.shape[0], table.shape[1]
    seqs = _rows(seqs, N)
    n_out = len(seqs)
    ids = np.full((n_out, G, kslots), -1, np.int32)
    gap = np.full((n_out, G), np.nan, np.float32)
    out = np.zeros((n_out, H, d), np.float64)
    pages = [_pages_of(table, lens, n, B, npages) for n in seqs]
    valid = np.array([p is not None for p in pages], bool)
    vr = np.nonzero(valid)[0]
    if len(vr) == 0:
        return ids, gap, out, valid
    # gather the valid sequences' pages, in logical order, into one contiguous batch
    Lc = max(len(pages[r]) for r in vr) * B
    kc = np.zeros((len(vr), Lc, G, d), np.uint16)
    vc = np.zeros((len(vr), Lc, G, d), np.uint16)
    ikc = np.zeros((len(vr), Lc, dI), np.uint16)
    for j, r in enumerate(vr):
        n_tok = len(pages[r]) * B
        kc[j, :n_tok] = kp[pages[r]].reshape(n_tok, G, d)
        vc[j, :n_tok] = vp[pages[r]].reshape(n_tok, G, d)
        ikc[j, :n_tok] = ikp[pages[r]].reshape(n_tok, dI)
    sv = seqs[vr]
    ids[vr], gap[vr], out[vr] = decode(q[sv], iq[sv], kc, vc, ikc, lens[sv], B, kslots, scale,
                                       lib=lib)
    return ids, gap, out, valid


def _pages_of(table, lens, n, B, npages):
    """Page ids of sequence n's blocks 0 .. (len-1)/B in logical order, or None when
    the length is outside [1, max_blocks * B] or a page id is outside the pool."""
    Ln = int(lens[n])
    if Ln < 1 or Ln > table.shape[1] * B:
        return None
    pages = table[n, :(Ln - 1) // B + 1]
    if pages.min() < 0 or pages.max() >= npages:
        return None
    return pages


def decode_paged_attend(q, k_pages, v_pages, block_table, seq_len, ids, B, scale, seqs,
                        lib=None):
    """Paged decode main branch for the listed (valid) sequences with given ids."""
    q, kp, vp = _u16(q), _u16(k_pages), _u16(v_pages)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                       dtype=np.int64)
    lens = np.asarray(seq_len.cpu() if hasattr(seq_len, "cpu") else seq_len, dtype=np.int64)
    N, H, d = q.shape
    G = kp.shape[2]
    ids = np.asarray(ids, np.int32)
    out = np.zeros((len(seqs), H, d), np.float64)
    for r, n in enumerate(seqs):
        pages = _pages_of(table, lens, n, B, kp.shape[0])
        if pages is None:
            raise ValueError(f"sequence {n} is not valid")
        Lc = len(pages) * B
        out[r] = decode_attend(q[n:n + 1], kp[pages].reshape(1, Lc, G, d),
                               vp[pages].reshape(1, Lc, G, d), [int(lens[n])], ids[r:r + 1], B,
                               scale, [0], lib=lib)[0]
    return out


# --------------------------------------------------------------------------
# FP8 (OCP E4M3) index-key cache for decode
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_table(lib=None) -> np.ndarray:
    """Value of each of the 256 E4M3 bytes (NaN for the two NaN patterns)."""
    lib = lib or load()
    out = np.empty(256, np.float64)
    lib.oracle_e4m3_table(_ptr(out))
    return out


def quantize_e4m3_rows(x, lib=None):
    """Per-row power-of-two scaling + E4M3 rounding of bf16 rows [..., dI].

    For each row: amax = max |x|; scale = 2^e with e the smallest integer such
    that amax <= 448 * 2^e (e = 0 for an all-zero row); every element is x / scale
    (exact) rounded to the nearest E4M3 value, ties to the even code (last bit 0);
    the sign bit is the sign of x.  Returns (bytes uint8 [..., dI], scale fp32 [...]).
    """
    table = e4m3_table(lib)
    mags = table[:127]                       # codes 0x00..0x7E: 0 .. 448 ascending
    xv = _u16(x).astype(np.uint32) << 16
    xf = xv.view(np.float32).astype(np.float64)
    amax = np.abs(xf).max(axis=-1)
    e = np.zeros(amax.shape, np.int64)
    nz = amax > 0
    # smallest e with amax <= 448 * 2^e
    m, ex = np.frexp(amax[nz] / E4M3_MAX)    # amax/448 = m * 2^ex, m in [0.5, 1)
    e[nz] = np.where(m == 0.5, ex - 1, ex)
    scale = np.ldexp(1.0, e)
    y = np.abs(xf) / scale[..., None]
    hi = np.searchsorted(mags, y, side="left").clip(0, 126)   # first value >= y
    lo = (hi - 1).clip(0, 126)
    d_hi = mags[hi] - y
    d_lo = y - mags[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code |= (np.signbit(xf).astype(np.uint8) << 7)
    return code, scale.astype(np.float32)


def decode_fp8idx(q, iq, k_cache, v_cache, ik8, kscale, seq_len, B, kslots, scale=None,
                  seqs=None, lib=None):
    """Decode with an E4M3 index-key cache: (ids, gap, out)."""
    lib = lib or load()
    q, iq = _u16(q), _u16(iq)
    kc, vc = _u16(k_cache), _u16(v_cache)
    ik8 = np.ascontiguousarray(ik8.cpu().numpy() if hasattr(ik8, "cpu") else ik8, np.uint8)
    ks = np.ascontiguousarray(kscale.cpu().numpy() if hasattr(kscale, "cpu") else kscale,
                              np.float32)
    N, H, d = q.shape
    G, dI = iq.shape[1], iq.shape[2]
    Lmax = kc.shape[1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    seq_len = np.ascontiguousarray(np.asarray(seq_len, dtype=np.int64))
    seqs = _rows(seqs, N)
    n = len(seqs)
    ids = np.empty((n, G, kslots), np.int32)
    gap = np.empty((n, G), np.float32)
    out = np.empty((n, H, d), np.float64)
    lib.oracle_decode_fp8idx(_ptr(q), _ptr(iq), _ptr(kc), _ptr(vc), _ptr(ik8), _ptr(ks),
                             _ptr(seq_len), Lmax, H, G, d, dI, B, kslots, float(scale),
                             _ptr(seqs), n, _ptr(ids), _ptr(gap), _ptr(out))
    return ids, gap, out


def decode_paged_fp8idx(q, iq, k_pages, v_pages, ik8_pages, ksc_pages, block_table, seq_len, B,
                        kslots, scale=None, seqs=None, lib=None):
    """Paged decode with E4M3 index-key pages: (ids, gap, out, valid).

    The listed sequences' pages (K, V, E4M3 index bytes and their scales) are
    gathered in logical order into contiguous caches and decode_fp8idx runs on
    them; invalid sequences as in decode_paged.
    """
    q, iq = _u16(q), _u16(iq)
    kp, vp = _u16(k_pages), _u16(v_pages)
    ik8p = np.ascontiguousarray(ik8_pages.cpu().numpy() if hasattr(ik8_pages, "cpu")
                                else ik8_pages, np.uint8)
    kscp = np.ascontiguousarray(ksc_pages.cpu().numpy() if hasattr(ksc_pages, "cpu")
                                else ksc_pages, np.float32)
    table = np.asarray(block_table.cpu() if hasattr(block_table, "cpu") else block_table,
                       dtype=np.int64)
    lens = np.asarray(seq_len.cpu() if hasattr(seq_len, "cpu") else seq_len, dtype=np.int64)
    N, H, d = q.shape
    G, dI = iq.shape[1], iq.shape[2]
    seqs = _rows(seqs, N)
    n_out = len(seqs)
    ids = np.full((n_out, G, kslots), -1, np.int32)
    gap = np.full((n_out, G), np.nan, np.float32)
    out = np.zeros((n_out, H, d), np.float64)
    pages = [_pages_of(table, lens, n, B, kp.shape[0]) for n in seqs]
    valid = np.array([p is not None for p in pages], bool)
    vr = np.nonzero(valid)[0]
    if len(vr) == 0:
        return ids, gap, out, valid
    Lc = max(len(pages[r]) for r in vr) * B
    kc = np.zeros((len(vr), Lc, G, d), np.uint16)
    vc = np.zeros((len(vr), Lc, G, d), np.uint16)
    ik8 = np.zeros((len(vr), Lc, dI), np.uint8)
    ksc = np.ones((len(vr), Lc), np.float32)
    for j, r in enumerate(vr):
        n_tok = len(pages[r]) * B
        kc[j, :n_tok] = kp[pages[r]].reshape(n_tok, G, d)
        vc[j, :n_tok] = vp[pages[r]].reshape(n_tok, G, d)
        ik8[j, :n_tok] = ik8p[pages[r]].reshape(n_tok, dI)
        ksc[j, :n_tok] = kscp[pages[r]].reshape(n_tok)
    sv = seqs[vr]
    ids[vr], gap[vr], out[vr] = decode_fp8idx(q[sv], iq[sv], kc, vc, ik8, ksc, lens[sv], B,
                                              kslots, scale, lib=lib)
    return ids, gap, out, valid
