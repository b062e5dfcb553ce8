"""HIP-graph capture of the library's entry points (a serving loop replays one
captured step per token).  The calls allocate nothing, synchronise nothing and
record no memset, so a step captured once (outputs and workspace allocated
beforehand) replays correctly.  Every replay follows eager work on the same
buffers (the outputs are overwritten, the inputs changed in place) and must equal
a fresh eager call on the same inputs bitwise."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _say(msg):
    print(f"[graphs] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_long_idx_amd as msa  # noqa: F401  (fails loudly if not built)
    msa.load_library()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    """Run fn once eagerly on a side stream (warm-up), then capture it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays(g, outs, eager, mutate, n=3):
    """n replays, each after eager work: mutate the inputs, scribble over the
    outputs; every replay must equal eager() on the mutated inputs."""
    for r in range(n):
        mutate(r)
        for o in outs:
            o.fill_(-1 if o.dtype == torch.int32 else float("nan"))
        junk = torch.randn(512, 512, device=DEV) @ torch.randn(512, 512, device=DEV)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        want = eager()
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else b), \
                f"replay {r} differs from the eager call"
        del junk
        _say(f"  replay {r}: equal to the eager call")


def test_decode_step_graph():
    """Decode of 8 sequences captured once; the replays see new query rows and
    longer sequences, as a token loop would."""
    import block_sparse_long_idx_amd as msa
    s = synth.DecodeShape(N=8, Lc=3000, H=16, G=4, d=128, dI=128, B=128, k=8)
    x = synth.decode_inputs(s, seed=70, device=DEV)
    lens0 = np.asarray(x["seq_len"], np.int32)
    sl = torch.tensor(lens0, device=DEV)
    out = torch.empty_like(x["q"])
    ids = torch.empty((s.N, s.G, s.k), dtype=torch.int32, device=DEV)
    ws = msa._workspace(msa.workspace_size("decode", N=s.N, Lmax=s.Lc, H=s.H, G=s.G, d=s.d,
                                           dI=s.dI, k=s.k), DEV)

    def step():
        msa.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"], sl, kslots=s.k,
                   out=out, ids_out=ids, workspace=ws, return_ids=True)

    def eager():
        return msa.decode(x["q"], x["iq"], x["k_cache"], x["v_cache"], x["ik_cache"], sl,
                          kslots=s.k, return_ids=True)

    def mutate(r):
        g_ = torch.Generator(device=DEV).manual_seed(100 + r)
        x["q"].copy_(torch.randn(x["q"].shape, device=DEV, generator=g_).to(torch.bfloat16))
        sl.copy_(torch.tensor(np.minimum(lens0 + 37 * (r + 1), s.Lc), device=DEV))

    _say("decode step")
    g = _capture(step)
    _replays(g, [out, ids], eager, mutate)


def test_prefill_graph():
    """Prefill of L = 5000 captured once; the replays see new q and index rows."""
    import block_sparse_long_idx_amd as msa
    s = synth.PrefillShape(L=5000, H=16, G=4, d=128, dI=128, B=128, k=8)
    x = {n: t.to(DEV) for n, t in synth.prefill_inputs(s, seed=71).items()
         if isinstance(t, torch.Tensor)}
    out = torch.empty_like(x["q"])
    ids = torch.empty((s.L, s.G, s.k), dtype=torch.int32, device=DEV)
    ws = msa._workspace(msa.workspace_size("prefill", L=s.L, H=s.H, G=s.G, d=s.d, dI=s.dI,
                                           k=s.k), DEV)

    def step():
        msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=s.k, out=out, ids_out=ids,
                    workspace=ws, return_ids=True)

    def eager():
        return msa.prefill(x["q"], x["k"], x["v"], x["iq"], x["ik"], kslots=s.k, return_ids=True)

    def mutate(r):
        g_ = torch.Generator(device=DEV).manual_seed(200 + r)
        for n in ("q", "iq"):
            x[n].copy_(torch.randn(x[n].shape, device=DEV, generator=g_).to(torch.bfloat16))

    _say("prefill L=5000")
    g = _capture(step)
    _replays(g, [out, ids], eager, mutate)


def test_batched_varlen_graph():
    """A batch of 20 short prompts captured once, at k = 2: those of at most 256
    tokens go to one dense-kernel launch, the runs of longer ones to K1..K5 batches."""
    import block_sparse_long_idx_amd as msa
    kw = dict(H=16, G=4, d=128, dI=128, k=2)
    lens = [1, 127, 128, 129, 300, 511, 640, 700, 50, 200, 333, 64, 600, 256, 257, 90, 10, 400,
            512, 128]
    parts = [synth.prefill_inputs(synth.PrefillShape(L=L, B=128, **kw), seed=300 + i)
             for i, L in enumerate(lens)]
    c = {n: torch.cat([p[n] for p in parts]).to(DEV) for n in ("q", "k", "v", "iq", "ik")}
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    out = torch.empty_like(c["q"])
    ids = torch.empty((cu[-1], kw["G"], kw["k"]), dtype=torch.int32, device=DEV)
    ws = msa._workspace(msa.workspace_size("prefill_varlen", cu_q=cu, cu_kv=cu, **kw), DEV)

    def step():
        msa.prefill_varlen(c["q"], c["k"], c["v"], c["iq"], c["ik"], cu, cu, kslots=kw["k"],
                           out=out, ids_out=ids, workspace=ws, return_ids=True)

    def eager():
        return msa.prefill_varlen(c["q"], c["k"], c["v"], c["iq"], c["ik"], cu, cu,
                                  kslots=kw["k"], return_ids=True)

    def mutate(r):
        g_ = torch.Generator(device=DEV).manual_seed(400 + r)
        c["v"].copy_(torch.randn(c["v"].shape, device=DEV, generator=g_).to(torch.bfloat16))

    _say("batched varlen, 20 prompts")
    g = _capture(step)
    _replays(g, [out, ids], eager, mutate)


def test_paged_fp8_decode_graph():
    """Paged decode over E4M3 index pages captured once; the replays see a new
    query and a block table with pages swapped."""
    import block_sparse_long_idx_amd as msa
    s = synth.DecodeShape(N=6, Lc=2500, H=16, G=4, d=128, dI=128, B=128, k=8)
    x = synth.decode_inputs(s, seed=72, device=DEV)
    ik8, isc = msa.quantize_idx_k_e4m3(x["ik_cache"])
    x["ik8"], x["isc"] = ik8, isc
    pg = synth.paginate(x, 128, seed=73, names=("k_cache", "v_cache", "ik8", "isc"))
    table = pg["block_table"].to(DEV)
    sl = torch.tensor(np.asarray(x["seq_len"], np.int32), device=DEV)
    out = torch.empty_like(x["q"])
    ids = torch.empty((s.N, s.G, s.k), dtype=torch.int32, device=DEV)
    ws = msa._workspace(msa.workspace_size("decode_paged", N=s.N, max_blocks=table.shape[1],
                                           H=s.H, G=s.G, d=s.d, dI=s.dI, k=s.k), DEV)
    args = lambda: (x["q"], x["iq"], pg["k_pages"], pg["v_pages"],  # noqa: E731
                    pg["ik8_pages"], pg["isc_pages"], table, sl)

    def step():
        msa.decode_paged_fp8idx(*args(), kslots=s.k, out=out, ids_out=ids, workspace=ws,
                                return_ids=True)

    def eager():
        return msa.decode_paged_fp8idx(*args(), kslots=s.k, return_ids=True)

    def mutate(r):
        g_ = torch.Generator(device=DEV).manual_seed(500 + r)
        x["q"].copy_(torch.randn(x["q"].shape, device=DEV, generator=g_).to(torch.bfloat16))
        t = table.clone()
        table[:, [0, 1]] = t[:, [1, 0]]          # two blocks of every sequence change pages

    _say("paged E4M3 decode")
    g = _capture(step)
    _replays(g, [out, ids], eager, mutate)
