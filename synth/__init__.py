"""Seeded synthetic inputs for the MSA forward pass.

This module holds no arithmetic of the method itself: it only draws bf16
tensors with the shapes, value distribution and planted structure of the
workloads, on the CPU or directly on a GPU.  Both the HIP path's tests and the
oracle consume exactly the bytes it returns.

Distribution: every tensor is N(0,1) drawn in fp32 and rounded once to bf16.
Large tensors are drawn in row chunks, each chunk from its own generator seeded
by (seed, tensor id, chunk index), so any chunk can be regenerated on its own.

Planting (so that selection is not tie-dominated, and to create hot blocks):

* ``"lit"`` -- the recipe as the workload text states it: per group g,
  ``u_g = normalize(mean_i iq[i,g,:])`` and ``c * u_g`` is added to the idx-K
  rows of ``n_plant`` randomly chosen blocks per group.  Because idx-Q has zero
  mean this barely changes which blocks win; it is kept because it is the
  literal reading.
* ``"hot"`` -- a seeded unit vector ``u_g`` per group is made the real idx-Q
  mean (``iq[:,g,:] += 8 u_g``) and ``c * sqrt(dI) * u_g`` is added to the
  planted idx-K rows, so planted blocks are selected by (nearly) every query.
  (The query's own N(0,1) part projected on the planted vector is shared by
  every token of a planted block; a mean of 8 keeps that term at about a
  quarter of the planted signal.)
  With ``hot_blocks=(0,1,2,3)`` every group's direction is added to those
  blocks: the long-context skewed workload.
* ``"none"`` -- plain N(0,1).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

_CHUNK_ELEMS = 1 << 26  # elements drawn per generator chunk (256 MiB of fp32)

T_Q, T_K, T_V, T_IQ, T_IK, T_PLANT, T_IDS = 1, 2, 3, 4, 5, 6, 7
HOT_MEAN = 8.0   # strength of the group mean direction in idx-Q for "hot" planting


@dataclass(frozen=True)
class PrefillShape:
    L: int
    H: int
    G: int
    d: int
    dI: int
    B: int = 128
    k: int = 16


@dataclass(frozen=True)
class DecodeShape:
    N: int
    Lc: int
    H: int
    G: int
    d: int
    dI: int
    B: int = 128
    k: int = 16


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "prefill_varlen" | "sparse_attn" | "decode" |
                              # "decode_paged" | "decode_fp8idx" | "decode_paged_fp8idx"
    shape: object
    plant: str = "lit"
    n_plant: int = 4
    c: float = 2.0
    hot_blocks: tuple = field(default_factory=tuple)
    batch: int = 1            # prefill_varlen: sequences of shape.L tokens packed in one call
    chunk: int = 0            # prefill_varlen: new tokens per call over the growing prefix (0: all)


# The five workloads: shapes of the pages' research model (64 query heads,
# 4 KV heads, B = 128, k = 16) with head/index dims 128, plus the tiny case; and
# the decode workload again, with its caches in shuffled 128-token pages, and with
# its index-key cache held as E4M3 bytes plus per-token scales; and packed /
# chunked prefills (8 sequences of 16384 tokens in one call; 256 prompts of 512
# tokens in one call; the 128K sequence prefilled 16384 new tokens at a time over
# its growing cached prefix).
WORKLOADS = {
    "tiny_prefill_L4096": Workload("tiny_prefill_L4096", "prefill",
                                   PrefillShape(L=4096, H=8, G=2, d=64, dI=32, B=128, k=4)),
    "prefill_L32768": Workload("prefill_L32768", "prefill",
                               PrefillShape(L=32768, H=64, G=4, d=128, dI=128)),
    "prefill_L131072": Workload("prefill_L131072", "prefill",
                                PrefillShape(L=131072, H=64, G=4, d=128, dI=128)),
    # the main branch alone on constructed skewed ids: blocks 0-3 + own block + 11
    # random distinct blocks per (query, group), so blocks 0-3 are hot KV tiles
    "sparse_attn_L131072_skewed": Workload("sparse_attn_L131072_skewed", "sparse_attn",
                                           PrefillShape(L=131072, H=64, G=4, d=128, dI=128),
                                           plant="none", hot_blocks=(0, 1, 2, 3)),
    "decode_N64_L262144": Workload("decode_N64_L262144", "decode",
                                   DecodeShape(N=64, Lc=262144, H=64, G=4, d=128, dI=128)),
    "prefill_L1048576_hot": Workload("prefill_L1048576_hot", "prefill",
                                     PrefillShape(L=1048576, H=64, G=4, d=128, dI=128),
                                     plant="hot", n_plant=0, c=3.0, hot_blocks=(0, 1, 2, 3)),
    "prefill_varlen_8x16384": Workload("prefill_varlen_8x16384", "prefill_varlen",
                                       PrefillShape(L=16384, H=64, G=4, d=128, dI=128), batch=8),
    "prefill_varlen_256x512": Workload("prefill_varlen_256x512", "prefill_varlen",
                                       PrefillShape(L=512, H=64, G=4, d=128, dI=128), batch=256),
    "prefill_chunked_L131072_C16384": Workload("prefill_chunked_L131072_C16384", "prefill_varlen",
                                               PrefillShape(L=131072, H=64, G=4, d=128, dI=128),
                                               chunk=16384),
    "decode_paged_N64_L262144": Workload("decode_paged_N64_L262144", "decode_paged",
                                         DecodeShape(N=64, Lc=262144, H=64, G=4, d=128,
                                                     dI=128)),
    "decode_fp8idx_N64_L262144": Workload("decode_fp8idx_N64_L262144", "decode_fp8idx",
                                          DecodeShape(N=64, Lc=262144, H=64, G=4, d=128,
                                                      dI=128)),
    "decode_paged_fp8idx_N64_L262144": Workload("decode_paged_fp8idx_N64_L262144",
                                                "decode_paged_fp8idx",
                                                DecodeShape(N=64, Lc=262144, H=64, G=4, d=128,
                                                            dI=128)),
}


def _seed(seed: int, tid: int, chunk: int) -> int:
    # distinct 63-bit generator seeds per (seed, tensor, chunk)
    x = (seed * 0x9E3779B1 + tid * 0x85EBCA77 + chunk * 0xC2B2AE3D) & ((1 << 63) - 1)
    return x or 1


def randn_fp32(shape, seed: int, tid: int, device) -> torch.Tensor:
    """N(0,1) fp32 tensor drawn in row chunks (dim 0) from per-chunk generators."""
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows_per = max(1, _CHUNK_ELEMS // max(row, 1))
    for ci, r0 in enumerate(range(0, shape[0], rows_per)):
        r1 = min(shape[0], r0 + rows_per)
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, tid, ci))
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=g, device=device,
                                 dtype=torch.float32)
    return out


def randn_bf16(shape, seed: int, tid: int, device) -> torch.Tensor:
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    row = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows_per = max(1, _CHUNK_ELEMS // max(row, 1))
    for ci, r0 in enumerate(range(0, shape[0], rows_per)):
        r1 = min(shape[0], r0 + rows_per)
        g = torch.Generator(device=device)
        g.manual_seed(_seed(seed, tid, ci))
        out[r0:r1] = torch.randn((r1 - r0,) + shape[1:], generator=g, device=device,
                                 dtype=torch.float32).to(torch.bfloat16)
    return out


def _unit_vectors(n: int, dim: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(_seed(seed, T_PLANT, 1))
    u = rng.standard_normal((n, dim))
    return u / np.linalg.norm(u, axis=1, keepdims=True)


def planted_blocks(nb: int, G: int, n_plant: int, seed: int) -> np.ndarray:
    """[G, n_plant] distinct block ids per group (seeded host draw)."""
    rng = np.random.default_rng(_seed(seed, T_PLANT, 2))
    n_plant = min(n_plant, nb)
    return np.stack([rng.choice(nb, size=n_plant, replace=False) for _ in range(G)]) \
        if n_plant > 0 else np.zeros((G, 0), np.int64)


def prefill_inputs(shape: PrefillShape, seed: int, plant: str = "lit", n_plant: int = 4,
                   c: float = 2.0, hot_blocks=(), device="cpu") -> dict:
    """q[L,H,d], k[L,G,d], v[L,G,d], iq[L,G,dI], ik[L,dI] as bf16 tensors on `device`."""
    s = shape
    nb = (s.L + s.B - 1) // s.B
    out = {
        "q": randn_bf16((s.L, s.H, s.d), seed, T_Q, device),
        "k": randn_bf16((s.L, s.G, s.d), seed, T_K, device),
        "v": randn_bf16((s.L, s.G, s.d), seed, T_V, device),
    }
    ik = randn_fp32((s.L, s.dI), seed, T_IK, device)
    if plant == "hot":
        u = torch.tensor(_unit_vectors(s.G, s.dI, seed), dtype=torch.float32, device=device)
        iq32 = randn_fp32((s.L, s.G, s.dI), seed, T_IQ, device)
        iq32 += HOT_MEAN * u[None, :, :]
        iq = iq32.to(torch.bfloat16)
        del iq32
        amp = c * math.sqrt(s.dI)
    elif plant == "lit":
        iq = randn_bf16((s.L, s.G, s.dI), seed, T_IQ, device)
        mean = iq.float().mean(dim=0)                       # [G, dI]
        u = mean / mean.norm(dim=1, keepdim=True).clamp_min(1e-30)
        amp = c
    elif plant == "none":
        iq = randn_bf16((s.L, s.G, s.dI), seed, T_IQ, device)
        u, amp = None, 0.0
    else:
        raise ValueError(f"unknown planting {plant!r}")
    blocks = np.zeros((s.G, 0), np.int64)
    if u is not None:
        blocks = planted_blocks(nb, s.G, n_plant, seed)
        for g in range(s.G):
            for b in blocks[g]:
                ik[b * s.B:min(s.L, (b + 1) * s.B)] += amp * u[g]
        for b in hot_blocks:
            for g in range(s.G):
                ik[b * s.B:min(s.L, (b + 1) * s.B)] += amp * u[g]
    out["iq"] = iq
    out["ik"] = ik.to(torch.bfloat16)
    out["planted"] = blocks
    return out


def decode_inputs(shape: DecodeShape, seed: int, plant: str = "lit", n_plant: int = 4,
                  c: float = 2.0, seq_len=None, device="cpu") -> dict:
    """q[N,H,d], iq[N,G,dI], k_cache/v_cache[N,Lc,G,d], ik_cache[N,Lc,dI], seq_len[N].

    With planting "lit" each sequence's query direction normalize(iq[n,g]) is
    added (times c) to the idx-K rows of n_plant random non-local blocks per group.
    """
    s = shape
    if seq_len is None:
        seq_len = np.full(s.N, s.Lc, np.int64)
    seq_len = np.asarray(seq_len, np.int64)
    out = {
        "q": randn_bf16((s.N, s.H, s.d), seed, T_Q, device),
        "iq": randn_bf16((s.N, s.G, s.dI), seed, T_IQ, device),
        "k_cache": randn_bf16((s.N, s.Lc, s.G, s.d), seed, T_K, device),
        "v_cache": randn_bf16((s.N, s.Lc, s.G, s.d), seed, T_V, device),
    }
    ik = randn_bf16((s.N, s.Lc, s.dI), seed, T_IK, device)
    rng = np.random.default_rng(_seed(seed, T_PLANT, 3))
    planted = []
    if plant == "lit" and n_plant > 0:
        for n in range(s.N):
            nbn = int((seq_len[n] - 1) // s.B)            # non-local blocks of this sequence
            row = []
            for g in range(s.G):
                if nbn == 0:
                    row.append([])
                    continue
                blk = rng.choice(nbn, size=min(n_plant, nbn), replace=False)
                u = out["iq"][n, g].float()
                u = u / u.norm().clamp_min(1e-30)
                for b in blk:
                    seg = ik[n, b * s.B:(b + 1) * s.B].float() + c * u
                    ik[n, b * s.B:(b + 1) * s.B] = seg.to(torch.bfloat16)
                row.append(list(blk))
            planted.append(row)
    elif plant not in ("lit", "none"):
        raise ValueError(f"unknown planting {plant!r}")
    out["ik_cache"] = ik
    out["seq_len"] = seq_len
    out["planted"] = planted
    return out


def skewed_ids(L: int, G: int, k: int, B: int = 128, hot: tuple = (0, 1, 2, 3), seed: int = 0,
               device="cpu") -> torch.Tensor:
    """Constructed block ids [L, G, k] int32 that make blocks ``hot`` hot KV tiles.

    Row (i, g) with b(i) = i // B >= k lists the hot blocks, the own block b(i) and
    k - 1 - len(hot) further blocks drawn uniformly without replacement from
    [len(hot), b(i)); a row with b(i) < k lists every block 0 .. b(i) and pads with
    -1.  Ids ascending.  Drawn in row chunks from per-(seed, chunk) generators.
    """
    nb = (L + B - 1) // B
    nh = len(hot)
    if tuple(hot) != tuple(range(nh)) or k < nh + 2:
        raise ValueError("hot blocks must be 0 .. n-1 with n + 2 <= k")
    m = k - 1 - nh
    out = torch.empty((L, G, k), dtype=torch.int32, device=device)
    blk = torch.arange(nb, device=device)
    slot = torch.arange(k, device=device)
    rows_per = max(1, (1 << 24) // (G * nb))
    for ci, r0 in enumerate(range(0, L, rows_per)):
        r1 = min(L, r0 + rows_per)
        gen = torch.Generator(device=device)
        gen.manual_seed(_seed(seed, T_IDS, ci))
        bi = torch.arange(r0, r1, device=device) // B
        key = torch.rand((r1 - r0, G, nb), generator=gen, device=device)
        cand = (blk[None, :] >= nh) & (blk[None, :] < bi[:, None])
        key = torch.where(cand[:, None, :], key, torch.full_like(key, 2.0))
        drawn = torch.topk(key, m, dim=2, largest=False).indices
        fixed = torch.cat([blk[:nh].expand(r1 - r0, G, nh), bi[:, None, None].expand(r1 - r0, G, 1)],
                          dim=2)
        long_rows = torch.sort(torch.cat([fixed, drawn], dim=2), dim=2).values
        short_rows = torch.where(slot[None, :] <= bi[:, None], slot[None, :],
                                 torch.full_like(slot[None, :], -1))[:, None, :].expand(r1 - r0, G, k)
        out[r0:r1] = torch.where((bi >= k)[:, None, None], long_rows, short_rows).to(torch.int32)
    return out


def paginate(x: dict, B: int, seed: int, extra_pages: int = 0,
             names=("k_cache", "v_cache", "ik_cache")) -> dict:
    """Re-lay per-sequence caches [N, Lc, ...] (default: those of ``decode_inputs``)
    as B-token pages, every cache with the same page order.

    Logical block b of sequence n goes to page ``block_table[n, b]``; the pages are
    a seeded random permutation of all N * ceil(Lc / B) blocks, followed by
    ``extra_pages`` pages that no table entry names (N(0,1) for bf16 caches, zero
    otherwise).  A cache whose length is not a multiple of B is zero-padded to whole
    pages.  Returns, for each cache "<x>_cache" or "<x>", a pages tensor
    "<x>_pages" [P, B, ...] on the caches' device, and block_table [N, ceil(Lc / B)]
    (int32).
    """
    first = x[names[0]]
    N, Lc = first.shape[0], first.shape[1]
    nblk = (Lc + B - 1) // B
    pad = nblk * B - Lc
    dev = first.device
    gen = torch.Generator().manual_seed(_seed(seed, T_PLANT, 7))
    perm = torch.randperm(N * nblk, generator=gen).to(dev)
    P = N * nblk + extra_pages

    def lay(cache, tid):
        row_shape = tuple(cache.shape[2:])
        if extra_pages and cache.dtype == torch.bfloat16:
            pages = randn_bf16((P, B) + row_shape, seed, tid, dev)
        else:
            pages = torch.zeros((P, B) + row_shape, dtype=cache.dtype, device=dev)
        blocks = cache
        if pad:
            blocks = torch.cat([cache, torch.zeros((N, pad) + row_shape, dtype=cache.dtype,
                                                   device=dev)], dim=1)
        pages[perm] = blocks.reshape((N * nblk, B) + row_shape)
        return pages

    out = {"block_table": perm.view(N, nblk).to(torch.int32)}
    for i, name in enumerate(names):
        key = (name[:-len("_cache")] if name.endswith("_cache") else name) + "_pages"
        out[key] = lay(x[name], 11 + i)
    return out
