"""Forward and backward captured in a HIP graph (torch.cuda.CUDAGraph):
the library issues only kernel launches on the caller's stream (no memsets,
no allocations, no synchronisation), so a captured graph must reproduce the
eager results bit for bit on every replay.  Eager work and synchronisations
run between the replays."""
import pytest
import torch

import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _run(q, k, v, do, spec, bm):
    o, lse = fa.forward(q, k, v, return_lse=True, block_mask=bm, **spec)
    dq, dk, dv = fa.backward(q, k, v, o, do, lse, block_mask=bm, **spec)
    return o, lse, dq, dk, dv


@pytest.mark.parametrize("name", ["causal_alibi", "document_block_mask", "window_softcap"])
def test_graph_replays_match_eager(name):
    B, Hq, Hkv, S, D = 1, 4, 2, 600, 128
    q, k, v = (dev(t) for t in synth.qkv(B, Hq, Hkv, S, S, D, 60))
    do = dev(synth.randn((B, Hq, S, D), 61))
    bm = None
    if name == "causal_alibi":
        spec = dict(mask=fa.MASK_CAUSAL, mod=fa.MOD_ALIBI)
    elif name == "window_softcap":
        spec = dict(mask=fa.MASK_SLIDING_WINDOW, window=100, mod=fa.MOD_SOFTCAP, softcap=30.0)
    else:
        lens = synth.doc_lengths(S, 50, 300, 62)
        doc = dev(torch.from_numpy(synth.doc_ids_from_lengths(lens))[None])
        spec = dict(mask=fa.MASK_DOCUMENT, doc_ids=doc)
        bm = fa.build_block_mask(fa.MASK_DOCUMENT, B, S, S, doc_ids=doc)
    ref = _run(q, k, v, do, spec, bm)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _run(q, k, v, do, spec, bm)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = _run(q, k, v, do, spec, bm)
    for rep in range(3):
        for t in out:
            t.fill_(float("nan"))  # a replay must rewrite every element
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want, what in zip(out, ref, ("O", "LSE", "dQ", "dK", "dV")):
            assert torch.equal(got, want), (name, rep, what)
        _run(q, k, v, do, spec, bm)  # eager work between replays
        torch.cuda.synchronize()
