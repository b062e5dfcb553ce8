"""MiniMax Sparse Attention (MSA) forward pass on MI355X -- Python binding.

A thin ctypes layer over ``libmsa.so`` (C ABI in ``include/msa.h``): it checks
tensor dtypes/shapes/devices, allocates outputs and the workspace with torch,
passes raw device pointers and torch's current HIP stream, and turns status
codes into exceptions.  Every step of the computation runs in the library's
HIP kernels; there is no fallback path.  If the library is not built, every call
raises ``MSAError``.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["MSAError", "select_blocks", "sparse_attn", "prefill", "prefill_varlen", "decode",
           "decode_paged",
           "decode_fp8idx", "decode_paged_fp8idx", "quantize_idx_k_e4m3", "workspace_size",
           "library_path", "load_library", "timing_enable", "timing_collect", "timing_disable"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmsa.so")
_lib = None

MSA_OK = 0
_STATUS = {0: "MSA_OK", 1: "MSA_ERR_INVALID_ARG", 2: "MSA_ERR_UNSUPPORTED",
           3: "MSA_ERR_WORKSPACE_TOO_SMALL", 4: "MSA_ERR_HIP"}


class MSAError(RuntimeError):
    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


class _KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int),
                ("total_ms", ctypes.c_double)]


def timing_enable(max_launches: int = 4096):
    """Start per-kernel HIP-event timing of every stage the library enqueues."""
    _check(load_library().msa_timing_enable(max_launches), "msa_timing_enable")


def timing_collect() -> dict:
    """Wait for the recorded stages; {stage: (launches, total_ms)}; clears the record."""
    lib = load_library()
    buf = (_KernelTime * 32)()
    n = ctypes.c_int(0)
    _check(lib.msa_timing_collect(buf, 32, ctypes.byref(n)), "msa_timing_collect")
    return {buf[i].name.decode(): (buf[i].launches, buf[i].total_ms) for i in range(n.value)}


def timing_disable():
    load_library().msa_timing_disable()


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmsa.so (built in-tree by ``build.py``); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise MSAError(f"{_LIB_PATH} is not built; run __graft_entry__.build() "
                       "(or python block_sparse_long_idx_amd/build.py)")
    lib = ctypes.CDLL(_LIB_PATH)
    P, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t,
                            ctypes.c_float)
    lib.msa_status_string.argtypes = [i32]
    lib.msa_status_string.restype = ctypes.c_char_p
    lib.msa_select_blocks_workspace_size.argtypes = [i64, i32, i32, i32, i32]
    lib.msa_select_blocks_workspace_size.restype = sz
    lib.msa_select_blocks.argtypes = [P, P, i64, i32, i32, i32, i32, P, P, sz, P]
    lib.msa_select_blocks.restype = i32
    lib.msa_sparse_attn_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
    lib.msa_sparse_attn_workspace_size.restype = sz
    lib.msa_sparse_attn.argtypes = [P, P, P, P, i64, i32, i32, i32, i32, i32, f32, P, P, sz, P]
    lib.msa_sparse_attn.restype = i32
    lib.msa_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, i32]
    lib.msa_prefill_workspace_size.restype = sz
    lib.msa_prefill.argtypes = [P, P, P, P, P, i64, i32, i32, i32, i32, i32, i32, f32, P, P, P,
                                sz, P]
    lib.msa_prefill.restype = i32
    lib.msa_decode_workspace_size.argtypes = [i32, i64, i32, i32, i32, i32, i32, i32]
    lib.msa_decode_workspace_size.restype = sz
    lib.msa_decode.argtypes = [P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32, f32, P,
                               P, P, sz, P]
    lib.msa_decode.restype = i32
    lib.msa_decode_static.argtypes = [P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32,
                                      f32, P, P, P]
    lib.msa_decode_static.restype = i32
    lib.msa_decode_paged_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32]
    lib.msa_decode_paged_workspace_size.restype = sz
    lib.msa_decode_paged.argtypes = [P, P, P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, i32,
                                     i32, f32, P, P, P, sz, P]
    lib.msa_decode_paged.restype = i32
    lib.msa_prefill_varlen.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32, i32, i32,
                                       f32, P, P, P, sz, P]
    lib.msa_prefill_varlen.restype = i32
    lib.msa_prefill_varlen_workspace_size.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32]
    lib.msa_prefill_varlen_workspace_size.restype = sz
    lib.msa_decode_fp8idx.argtypes = [P, P, P, P, P, P, P, i32, i64, i32, i32, i32, i32, i32, i32,
                                      f32, P, P, P, sz, P]
    lib.msa_decode_fp8idx.restype = i32
    lib.msa_decode_paged_fp8idx.argtypes = [P, P, P, P, P, P, i64, P, i32, P, i32, i32, i32, i32,
                                            i32, i32, i32, f32, P, P, P, sz, P]
    lib.msa_decode_paged_fp8idx.restype = i32
    lib.msa_quantize_idx_k_e4m3.argtypes = [P, i64, i32, P, P, P]
    lib.msa_quantize_idx_k_e4m3.restype = i32
    lib.msa_timing_enable.argtypes = [i32]
    lib.msa_timing_enable.restype = i32
    lib.msa_timing_collect.argtypes = [ctypes.POINTER(_KernelTime), i32, ctypes.POINTER(i32)]
    lib.msa_timing_collect.restype = i32
    lib.msa_timing_disable.argtypes = []
    lib.msa_timing_disable.restype = None
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != MSA_OK:
        raise MSAError(f"{what} failed: {_STATUS.get(status, status)}", status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, ndim, device=None):
    if not isinstance(t, torch.Tensor):
        raise MSAError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise MSAError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise MSAError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise MSAError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise MSAError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise MSAError(f"{name} must be contiguous")


def _workspace(nbytes: int, device) -> torch.Tensor:
    """uint8 device buffer whose data pointer is 256-byte aligned."""
    buf = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(int(nbytes), 1)]


def _scale(scale, d):
    return float(scale) if scale is not None else 1.0 / math.sqrt(d)


def workspace_size(kind: str, **kw) -> int:
    lib = load_library()
    if kind == "select":
        return lib.msa_select_blocks_workspace_size(kw["L"], kw["G"], kw["dI"], kw.get("B", 128),
                                                    kw["k"])
    if kind == "sparse_attn":
        return lib.msa_sparse_attn_workspace_size(kw["L"], kw["H"], kw["G"], kw["d"],
                                                  kw.get("B", 128), kw["k"])
    if kind == "prefill":
        return lib.msa_prefill_workspace_size(kw["L"], kw["H"], kw["G"], kw["d"], kw["dI"],
                                              kw.get("B", 128), kw["k"])
    if kind == "decode":
        return lib.msa_decode_workspace_size(kw["N"], kw["Lmax"], kw["H"], kw["G"], kw["d"],
                                             kw["dI"], kw.get("B", 128), kw["k"])
    if kind == "decode_paged":
        return lib.msa_decode_paged_workspace_size(kw["N"], kw["max_blocks"], kw["H"], kw["G"],
                                                   kw["d"], kw["dI"], kw.get("B", 128), kw["k"])
    if kind == "prefill_varlen":
        import numpy as np
        cq = np.ascontiguousarray(np.asarray(kw["cu_q"], dtype=np.int64))
        ckv = np.ascontiguousarray(np.asarray(kw["cu_kv"], dtype=np.int64))
        return lib.msa_prefill_varlen_workspace_size(cq.ctypes.data, ckv.ctypes.data, len(cq) - 1,
                                                     kw["H"], kw["G"], kw["d"], kw["dI"],
                                                     kw.get("B", 128), kw["k"])
    raise ValueError(kind)


def select_blocks(idx_q, idx_k, k: int = 16, B: int = 128, out=None, workspace=None):
    """Block ids [L, G, k] (int32, ascending, -1 padded) of the index branch."""
    lib = load_library()
    _need(idx_q, "idx_q", torch.bfloat16, 3)
    _need(idx_k, "idx_k", torch.bfloat16, 2, idx_q.device)
    L, G, dI = idx_q.shape
    if idx_k.shape != (L, dI):
        raise MSAError(f"idx_k must be [{L}, {dI}], got {tuple(idx_k.shape)}")
    if out is None:
        out = torch.empty((L, G, k), dtype=torch.int32, device=idx_q.device)
    _need(out, "out", torch.int32, 3, idx_q.device)
    nbytes = lib.msa_select_blocks_workspace_size(L, G, dI, B, k)
    ws = workspace if workspace is not None else _workspace(nbytes, idx_q.device)
    st = lib.msa_select_blocks(_ptr(idx_q), _ptr(idx_k), L, G, dI, B, k, _ptr(out), _ptr(ws),
                               ws.numel(), _stream(idx_q.device))
    _check(st, "msa_select_blocks")
    return out


def sparse_attn(q, k, v, block_ids, scale=None, B: int = 128, out=None, workspace=None):
    """Exact softmax attention over the listed blocks: out [L, H, d] bf16."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(k, "k", torch.bfloat16, 3, dev)
    _need(v, "v", torch.bfloat16, 3, dev)
    _need(block_ids, "block_ids", torch.int32, 3, dev)
    L, H, d = q.shape
    G = k.shape[1]
    kslots = block_ids.shape[2]
    if k.shape != (L, G, d) or v.shape != (L, G, d) or block_ids.shape[:2] != (L, G):
        raise MSAError("inconsistent shapes for q/k/v/block_ids")
    if out is None:
        out = torch.empty_like(q)
    nbytes = lib.msa_sparse_attn_workspace_size(L, H, G, d, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _ptr(block_ids), L, H, G, d, B, kslots,
                             _scale(scale, d), _ptr(out), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "msa_sparse_attn")
    return out


def prefill(q, k, v, idx_q, idx_k, kslots: int = 16, B: int = 128, scale=None,
            return_ids: bool = False, out=None, ids_out=None, workspace=None):
    """Whole MSA prefill: out [L, H, d] bf16 (and ids [L, G, k] if return_ids)."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    for name, t, nd in (("k", k, 3), ("v", v, 3), ("idx_q", idx_q, 3), ("idx_k", idx_k, 2)):
        _need(t, name, torch.bfloat16, nd, dev)
    L, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    if (k.shape != (L, G, d) or v.shape != (L, G, d) or idx_q.shape[0] != L
            or idx_k.shape != (L, dI)):
        raise MSAError("inconsistent shapes for q/k/v/idx_q/idx_k")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((L, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_prefill_workspace_size(L, H, G, d, dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(idx_q), _ptr(idx_k), L, H, G, d, dI, B,
                         kslots, _scale(scale, d), _ptr(out), _ptr(ids_out), _ptr(ws), ws.numel(),
                         _stream(dev))
    _check(st, "msa_prefill")
    return (out, ids_out) if return_ids else out


def decode(q, idx_q, k_cache, v_cache, idx_k_cache, seq_len, kslots: int = 16, B: int = 128,
           scale=None, return_ids: bool = False, out=None, ids_out=None, workspace=None):
    """MSA decode of N sequences (query = last cached token): out [N, H, d] bf16."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(idx_q, "idx_q", torch.bfloat16, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(idx_k_cache, "idx_k_cache", torch.bfloat16, 3, dev)
    _need(seq_len, "seq_len", torch.int32, 1, dev)
    N, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    Lmax = k_cache.shape[1]
    if (k_cache.shape != (N, Lmax, G, d) or v_cache.shape != (N, Lmax, G, d)
            or idx_k_cache.shape != (N, Lmax, dI) or seq_len.shape != (N,)):
        raise MSAError("inconsistent shapes for decode inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((N, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_decode_workspace_size(N, Lmax, H, G, d, dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_decode(_ptr(q), _ptr(idx_q), _ptr(k_cache), _ptr(v_cache), _ptr(idx_k_cache),
                        _ptr(seq_len), N, Lmax, H, G, d, dI, B, kslots, _scale(scale, d), _ptr(out),
                        _ptr(ids_out), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "msa_decode")
    return (out, ids_out) if return_ids else out


def decode_static(q, idx_q, k_cache, v_cache, idx_k_cache, seq_len, kslots: int = 16,
                  B: int = 128, scale=None, return_ids: bool = False, out=None, ids_out=None):
    """msa_decode without a caller workspace (the library's per-GPU static array of
    STATIC_SCRATCH_BYTES): same results as decode().  Pass out / ids_out to keep the
    call free of allocations."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(idx_q, "idx_q", torch.bfloat16, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(idx_k_cache, "idx_k_cache", torch.bfloat16, 3, dev)
    _need(seq_len, "seq_len", torch.int32, 1, dev)
    N, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    Lmax = k_cache.shape[1]
    if (k_cache.shape != (N, Lmax, G, d) or v_cache.shape != (N, Lmax, G, d)
            or idx_k_cache.shape != (N, Lmax, dI) or seq_len.shape != (N,)):
        raise MSAError("inconsistent shapes for decode inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((N, G, kslots), dtype=torch.int32, device=dev)
    st = lib.msa_decode_static(_ptr(q), _ptr(idx_q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(idx_k_cache), _ptr(seq_len), N, Lmax, H, G, d, dI, B, kslots,
                               _scale(scale, d), _ptr(out), _ptr(ids_out), _stream(dev))
    _check(st, "msa_decode_static")
    return (out, ids_out) if return_ids else out


# bytes of the per-GPU workspace array of decode_static (MSA_STATIC_SCRATCH_BYTES)
STATIC_SCRATCH_BYTES = 64 << 20


def decode_paged(q, idx_q, k_pages, v_pages, idx_k_pages, block_table, seq_len, kslots: int = 16,
                 B: int = 128, scale=None, return_ids: bool = False, out=None, ids_out=None,
                 workspace=None):
    """MSA decode over 128-token cache pages: out [N, H, d] bf16.

    k_pages/v_pages [P, 128, G, d], idx_k_pages [P, 128, dI]; block_table [N, max_blocks]
    int32 maps each sequence's logical block to its page.
    """
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(idx_q, "idx_q", torch.bfloat16, 3, dev)
    _need(k_pages, "k_pages", torch.bfloat16, 4, dev)
    _need(v_pages, "v_pages", torch.bfloat16, 4, dev)
    _need(idx_k_pages, "idx_k_pages", torch.bfloat16, 3, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_len, "seq_len", torch.int32, 1, dev)
    N, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    npages = k_pages.shape[0]
    maxb = block_table.shape[1]
    if (k_pages.shape != (npages, B, G, d) or v_pages.shape != (npages, B, G, d)
            or idx_k_pages.shape != (npages, B, dI) or block_table.shape[0] != N
            or seq_len.shape != (N,)):
        raise MSAError("inconsistent shapes for paged decode inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((N, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_decode_paged_workspace_size(N, maxb, H, G, d, dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_decode_paged(_ptr(q), _ptr(idx_q), _ptr(k_pages), _ptr(v_pages),
                              _ptr(idx_k_pages), npages, _ptr(block_table), maxb, _ptr(seq_len),
                              N, H, G, d, dI, B, kslots, _scale(scale, d), _ptr(out),
                              _ptr(ids_out), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "msa_decode_paged")
    return (out, ids_out) if return_ids else out


def quantize_idx_k_e4m3(idx_k, out=None, scale_out=None):
    """Index-key rows [..., dI] bf16 -> (E4M3 bytes [..., dI] uint8, scales [...] fp32)."""
    lib = load_library()
    if not isinstance(idx_k, torch.Tensor) or idx_k.dtype != torch.bfloat16 or not idx_k.is_cuda:
        raise MSAError("idx_k must be a bf16 GPU tensor")
    if not idx_k.is_contiguous():
        raise MSAError("idx_k must be contiguous")
    dI = idx_k.shape[-1]
    rows = idx_k.numel() // max(dI, 1)
    if out is None:
        out = torch.empty(idx_k.shape, dtype=torch.uint8, device=idx_k.device)
    if scale_out is None:
        scale_out = torch.empty(idx_k.shape[:-1], dtype=torch.float32, device=idx_k.device)
    st = lib.msa_quantize_idx_k_e4m3(_ptr(idx_k), rows, dI, _ptr(out), _ptr(scale_out),
                                     _stream(idx_k.device))
    _check(st, "msa_quantize_idx_k_e4m3")
    return out, scale_out


def decode_fp8idx(q, idx_q, k_cache, v_cache, idx_k_e4m3, idx_k_scale, seq_len, kslots: int = 16,
                  B: int = 128, scale=None, return_ids: bool = False, out=None, ids_out=None,
                  workspace=None):
    """MSA decode with an E4M3 index-key cache [N, Lmax, dI] (uint8) + scales [N, Lmax]."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(idx_q, "idx_q", torch.bfloat16, 3, dev)
    _need(k_cache, "k_cache", torch.bfloat16, 4, dev)
    _need(v_cache, "v_cache", torch.bfloat16, 4, dev)
    _need(idx_k_e4m3, "idx_k_e4m3", torch.uint8, 3, dev)
    _need(idx_k_scale, "idx_k_scale", torch.float32, 2, dev)
    _need(seq_len, "seq_len", torch.int32, 1, dev)
    N, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    Lmax = k_cache.shape[1]
    if (k_cache.shape != (N, Lmax, G, d) or v_cache.shape != (N, Lmax, G, d)
            or idx_k_e4m3.shape != (N, Lmax, dI) or idx_k_scale.shape != (N, Lmax)
            or seq_len.shape != (N,)):
        raise MSAError("inconsistent shapes for FP8 decode inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((N, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_decode_workspace_size(N, Lmax, H, G, d, dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_decode_fp8idx(_ptr(q), _ptr(idx_q), _ptr(k_cache), _ptr(v_cache),
                               _ptr(idx_k_e4m3), _ptr(idx_k_scale), _ptr(seq_len), N, Lmax, H, G,
                               d, dI, B, kslots, _scale(scale, d), _ptr(out), _ptr(ids_out),
                               _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "msa_decode_fp8idx")
    return (out, ids_out) if return_ids else out


def prefill_varlen(q, k, v, idx_q, idx_k, cu_q, cu_kv, kslots: int = 16, B: int = 128, scale=None,
                   return_ids: bool = False, out=None, ids_out=None, workspace=None):
    """Packed batch of causal sequences, each possibly continuing a cached prefix.

    q [sum C, H, d], idx_q [sum C, G, dI] hold the new tokens; k, v [sum L, G, d] and
    idx_k [sum L, dI] hold every token (prefix + new).  cu_q / cu_kv: offsets (host
    sequences of ints, nseq + 1 each).  Sequence s's prefix length L - C must be a
    multiple of 128.
    """
    import numpy as np
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    for name, t, nd in (("k", k, 3), ("v", v, 3), ("idx_q", idx_q, 3), ("idx_k", idx_k, 2)):
        _need(t, name, torch.bfloat16, nd, dev)
    cq = np.ascontiguousarray(np.asarray(cu_q, dtype=np.int64))
    ckv = np.ascontiguousarray(np.asarray(cu_kv, dtype=np.int64))
    nseq = len(cq) - 1
    if nseq < 0 or len(ckv) != nseq + 1:
        raise MSAError("cu_q and cu_kv must hold nseq + 1 offsets each")
    Tq, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    Tkv = k.shape[0]
    if (idx_q.shape[0] != Tq or k.shape != (Tkv, G, d) or v.shape != (Tkv, G, d)
            or idx_k.shape != (Tkv, dI) or (nseq > 0 and (cq[-1] > Tq or ckv[-1] > Tkv))):
        raise MSAError("inconsistent shapes for varlen prefill inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((Tq, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_prefill_varlen_workspace_size(cq.ctypes.data, ckv.ctypes.data, nseq, H, G, d,
                                                   dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_prefill_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(idx_q), _ptr(idx_k),
                                cq.ctypes.data, ckv.ctypes.data, nseq, H, G, d, dI, B, kslots,
                                _scale(scale, d), _ptr(out), _ptr(ids_out), _ptr(ws), ws.numel(),
                                _stream(dev))
    _check(st, "msa_prefill_varlen")
    return (out, ids_out) if return_ids else out


def decode_paged_fp8idx(q, idx_q, k_pages, v_pages, idx_k_pages_e4m3, idx_k_scale_pages,
                        block_table, seq_len, kslots: int = 16, B: int = 128, scale=None,
                        return_ids: bool = False, out=None, ids_out=None, workspace=None):
    """Paged decode with E4M3 index-key pages [P, 128, dI] (uint8) + scales [P, 128]."""
    lib = load_library()
    _need(q, "q", torch.bfloat16, 3)
    dev = q.device
    _need(idx_q, "idx_q", torch.bfloat16, 3, dev)
    _need(k_pages, "k_pages", torch.bfloat16, 4, dev)
    _need(v_pages, "v_pages", torch.bfloat16, 4, dev)
    _need(idx_k_pages_e4m3, "idx_k_pages_e4m3", torch.uint8, 3, dev)
    _need(idx_k_scale_pages, "idx_k_scale_pages", torch.float32, 2, dev)
    _need(block_table, "block_table", torch.int32, 2, dev)
    _need(seq_len, "seq_len", torch.int32, 1, dev)
    N, H, d = q.shape
    G, dI = idx_q.shape[1], idx_q.shape[2]
    npages = k_pages.shape[0]
    maxb = block_table.shape[1]
    if (k_pages.shape != (npages, B, G, d) or v_pages.shape != (npages, B, G, d)
            or idx_k_pages_e4m3.shape != (npages, B, dI)
            or idx_k_scale_pages.shape != (npages, B) or block_table.shape[0] != N
            or seq_len.shape != (N,)):
        raise MSAError("inconsistent shapes for paged FP8 decode inputs")
    if out is None:
        out = torch.empty_like(q)
    if return_ids and ids_out is None:
        ids_out = torch.empty((N, G, kslots), dtype=torch.int32, device=dev)
    nbytes = lib.msa_decode_paged_workspace_size(N, maxb, H, G, d, dI, B, kslots)
    ws = workspace if workspace is not None else _workspace(nbytes, dev)
    st = lib.msa_decode_paged_fp8idx(_ptr(q), _ptr(idx_q), _ptr(k_pages), _ptr(v_pages),
                                     _ptr(idx_k_pages_e4m3), _ptr(idx_k_scale_pages), npages,
                                     _ptr(block_table), maxb, _ptr(seq_len), N, H, G, d, dI, B,
                                     kslots, _scale(scale, d), _ptr(out), _ptr(ids_out), _ptr(ws),
                                     ws.numel(), _stream(dev))
    _check(st, "msa_decode_paged_fp8idx")
    return (out, ids_out) if return_ids else out
