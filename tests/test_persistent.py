"""The persistent, dynamically scheduled forward (fa_mask_params.work_queue):
workgroups take query tiles from counters in caller memory instead of one
workgroup per tile.  Only the order of tiles changes, so O and LSE must equal
the static schedule's bit for bit, the counters must be zero again after
every launch (the last workgroup clears them), and repeated launches and
graph replays must need no clearing in between."""
import pytest
import torch

import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import dev
from tests.test_fwd_parity import VARIANTS, doc_ids_for

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Sq, Skv, D, dtype, spec, seed, block_mask):
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, seed, dtype)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, seed + 1, dtype)
    doc = dev(doc_ids_for(B, Sq, seed)) if spec.get("mask") == 3 else None
    bm = None
    if block_mask:
        bm = fa.build_block_mask(spec.get("mask", 0), B, Sq, Skv, window=spec.get("window", 0), doc_ids=doc)
    return dev(q), dev(k), dev(v), doc, bm


CASES = [
    # (B, Hq, Hkv, Sq, Skv, D, dtype, variant, block mask)
    (2, 8, 4, 1300, 1300, 128, "bf16", "causal", False),   # 8 (batch, kv-head) units: one queue per XCD
    (1, 6, 3, 700, 700, 64, "bf16", "none_alibi", False),  # 3 units: a single queue
    (2, 4, 2, 333, 333, 128, "f32", "window", False),
    (1, 4, 4, 2000, 2000, 128, "bf16", "document", True),  # document mask, block-mask tile order
    (2, 8, 8, 900, 900, 128, "bf16", "document_alibi", True),
    (1, 16, 16, 1100, 1100, 128, "bf16", "causal_softcap_small", True),
    (1, 4, 2, 500, 333, 64, "bf16", "window_boost", False),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[7]}-{c[3]}-{c[6]}-bm{int(c[8])}" for c in CASES])
def test_persistent_matches_static_schedule(case):
    B, Hq, Hkv, Sq, Skv, D, dtype, name, block_mask = case
    spec = VARIANTS[name]
    q, k, v, doc, bm = _inputs(B, Hq, Hkv, Sq, Skv, D, dtype, spec, 40 + Sq, block_mask)
    o_ref, l_ref = fa.forward(q, k, v, doc_ids=doc, block_mask=bm, return_lse=True, **spec)
    wq = fa.new_work_queue()
    for rep in range(3):  # the queue is reused without clearing
        o, lse = fa.forward(q, k, v, doc_ids=doc, block_mask=bm, return_lse=True, work_queue=wq, **spec)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), (name, rep)
        assert torch.equal(lse, l_ref), (name, rep)
        assert int(wq.abs().sum()) == 0, wq.tolist()


def test_persistent_visits_every_tile_once():
    """The debug counters (key steps per query tile) equal the static
    schedule's: no tile is skipped or taken twice."""
    B, Hq, Hkv, S, D = 2, 8, 8, 1500, 128
    spec = VARIANTS["document"]
    q, k, v, doc, bm = _inputs(B, Hq, Hkv, S, S, D, "bf16", spec, 5, True)
    n_qt = -(-S // 128)
    ref = torch.zeros((B, Hq, n_qt), dtype=torch.int32, device="cuda")
    got = torch.zeros_like(ref)
    fa.forward(q, k, v, doc_ids=doc, block_mask=bm, visited=ref, **spec)
    fa.forward(q, k, v, doc_ids=doc, block_mask=bm, visited=got, work_queue=fa.new_work_queue(), **spec)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    assert int(ref.sum()) > 0


def test_persistent_graph_replays():
    """Captured in a HIP graph and replayed several times with eager work in
    between: the kernel clears its own queue, so every replay matches."""
    B, Hq, Hkv, S, D = 1, 8, 8, 1200, 128
    spec = VARIANTS["document"]
    q, k, v, doc, bm = _inputs(B, Hq, Hkv, S, S, D, "bf16", spec, 6, True)
    o_ref, l_ref = fa.forward(q, k, v, doc_ids=doc, block_mask=bm, return_lse=True, **spec)
    wq = fa.new_work_queue()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        o, lse = fa.forward(q, k, v, doc_ids=doc, block_mask=bm, return_lse=True, work_queue=wq, **spec)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.forward(q, k, v, doc_ids=doc, block_mask=bm, out=o, lse=lse, return_lse=True, work_queue=wq, **spec)
    for rep in range(3):
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), rep
        assert int(wq.abs().sum()) == 0
        fa.forward(q, k, v, doc_ids=doc, block_mask=bm, return_lse=True, work_queue=wq, **spec)  # eager, same queue
        torch.cuda.synchronize()
