"""Independent references used to pin the oracle (test helpers, CPU only).

These are deliberately written differently from the oracle: whole-matrix torch
fp64 operations and library attention (scaled_dot_product_attention with an
explicit mask) instead of per-row loops.
"""
from __future__ import annotations

import numpy as np
import torch


def f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().cpu().to(torch.float64)


def mask_from_ids(ids: np.ndarray, L: int, B: int, H: int, G: int) -> torch.Tensor:
    """Boolean attention mask [H, L, L]: query i may see key t iff block(t) is one
    of the ids of (i, group(h)) and t <= i."""
    r = H // G
    ids = torch.as_tensor(ids, dtype=torch.int64)            # [L, G, k]
    blk = torch.arange(L) // B                                # [L]
    sel = torch.zeros(L, G, (L + B - 1) // B, dtype=torch.bool)
    valid = ids >= 0
    ii, gg, ss = torch.nonzero(valid, as_tuple=True)
    sel[ii, gg, ids[ii, gg, ss]] = True
    allowed = sel[:, :, blk]                                  # [L(i), G, L(t)]
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    allowed = allowed & causal[:, None, :]
    return allowed.permute(1, 0, 2).repeat_interleave(r, dim=0)   # [H, L, L]


def sdpa_masked(q, k, v, mask, scale) -> torch.Tensor:
    """Library attention in fp64: q[L,H,d], k/v[L,G,d] (GQA), mask[H,L,L]."""
    H, G = q.shape[1], k.shape[1]
    r = H // G
    Q = f64(q).permute(1, 0, 2)                               # [H, L, d]
    K = f64(k).permute(1, 0, 2).repeat_interleave(r, dim=0)
    V = f64(v).permute(1, 0, 2).repeat_interleave(r, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=scale)
    return o.permute(1, 0, 2)                                 # [L, H, d]


def sdpa_causal(q, k, v, scale) -> torch.Tensor:
    H, G = q.shape[1], k.shape[1]
    r = H // G
    Q = f64(q).permute(1, 0, 2)
    K = f64(k).permute(1, 0, 2).repeat_interleave(r, dim=0)
    V = f64(v).permute(1, 0, 2).repeat_interleave(r, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=scale)
    return o.permute(1, 0, 2)


def softmax_pool_topk(iq, ik, B: int, k: int):
    """Selection taken the 'non exp-free' way: softmax over the causal token
    scores, max-pool the probabilities per block, library top-k over the
    competitors (blocks before the query's own), then add the own block.
    Returns ids [L, G, k] ascending, -1 padded."""
    IQ, IK = f64(iq), f64(ik)                                 # [L,G,dI], [L,dI]
    L, G, _ = IQ.shape
    nb = (L + B - 1) // B
    s = torch.einsum("igc,tc->git", IQ, IK)                   # [G, L, L] token scores
    causal = torch.tril(torch.ones(L, L, dtype=torch.bool))
    s = s.masked_fill(~causal, float("-inf"))
    p = torch.softmax(s, dim=-1)                              # fp64 probabilities
    pad = nb * B - L
    if pad:
        p = torch.nn.functional.pad(p, (0, pad))
    pooled = p.reshape(G, L, nb, B).amax(dim=-1)              # [G, L, nb]
    out = np.full((L, G, k), -1, np.int32)
    for i in range(L):
        bi = i // B
        for g in range(G):
            if bi <= k - 1:
                chosen = list(range(bi + 1))
            else:
                vals = pooled[g, i, :bi]
                top = torch.topk(vals, k - 1).indices.tolist()
                chosen = sorted(top + [bi])
            out[i, g, :len(chosen)] = chosen
    return out


def e4m3_rows_torch(x: torch.Tensor):
    """Per-row power-of-two scale + E4M3 rounding with torch's float8_e4m3fn cast
    (on whatever device x lives): (bytes uint8 [..., dI], scale fp32 [...]).
    Written independently of the oracle's table search, as a second route to the
    same bytes."""
    xf = x.float()
    amax = xf.abs().amax(dim=-1)
    m, ex = torch.frexp(amax / 448.0)
    e = torch.where(m == 0.5, ex - 1, ex)
    e = torch.where(amax > 0, e, torch.zeros_like(e))
    scale = torch.ldexp(torch.ones_like(amax), e)
    y = torch.ldexp(xf, -e[..., None].to(torch.float32))
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale
