"""Forward pass: HIP library against the fp64 oracle, element by element.

Shapes span several 128-row query tiles with ragged tails (S not a multiple
of the tile), both head dims, both dtypes, every mask and modifier, GQA and
MQA, Sq != Skv, the block-mask path, and the degenerate sizes.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import check_lse, check_out, dev, f32_scale

pytestmark = pytest.mark.gpu

VARIANTS = {
    "none": dict(mask=0),
    "causal": dict(mask=1),
    "window": dict(mask=2, window=77),
    "document": dict(mask=3),
    "causal_alibi": dict(mask=1, mod=1),
    "softcap": dict(mask=0, mod=2, softcap=30.0),
    "causal_softcap_small": dict(mask=1, mod=2, softcap=2.5),
    "boost": dict(mask=0, mod=3, boost_radius=128, boost_factor=1.1),
    "window_boost": dict(mask=2, window=200, mod=3, boost_radius=64, boost_factor=1.1),
    "document_alibi": dict(mask=3, mod=1),
    "none_alibi": dict(mask=0, mod=1),
    "window_softcap": dict(mask=2, window=130, mod=2, softcap=30.0),
}


def doc_ids_for(B, S, seed):
    ids = []
    for b in range(B):
        lens = synth.doc_lengths(S, 1, max(2, S // 3), seed + b)
        ids.append(synth.doc_ids_from_lengths(lens))
    return torch.from_numpy(np.stack(ids)).to(torch.int32)


def run_case(B, Hq, Hkv, Sq, Skv, D, dtype, spec, seed=0, rows=None, block_mask=False, return_lse=True):
    q, k, v = synth.qkv(B, Hq, Hkv, Sq, Skv, D, seed, dtype)
    scale = f32_scale(D)
    doc = doc_ids_for(B, Sq, seed) if spec.get("mask") == 3 else None
    var = oracle.Variant(doc_ids=None if doc is None else doc.numpy(), **spec)
    kw = {k_: v_ for k_, v_ in spec.items()}
    bm = None
    if block_mask:
        bm = fa.build_block_mask(spec.get("mask", 0), B, Sq, Skv, window=spec.get("window", 0), doc_ids=dev(doc))
    res = fa.forward(dev(q), dev(k), dev(v), scale=scale, doc_ids=dev(doc), return_lse=return_lse,
                     block_mask=bm, **kw)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(q, k, v, scale, var, rows=rows)
    return res, o_ref, l_ref


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_variants(name, D, dtype):
    (o, lse), o_ref, l_ref = run_case(2, 4, 2, 333, 333, D, dtype, VARIANTS[name], seed=11)
    check_out(o, o_ref, dtype)
    check_lse(lse, l_ref)


# Above 1024 keys the unmasked, causal and long-window forwards take the
# 8-wave ping-pong kernel (256-row tiles); every modifier at a size past that.
PP_VARIANTS = ["none", "causal", "causal_alibi", "softcap", "causal_softcap_small", "boost", "none_alibi"]


@pytest.mark.parametrize("name", PP_VARIANTS)
@pytest.mark.parametrize("D", [64, 128])
def test_variants_ping_pong_sizes(name, D):
    (o, lse), o_ref, l_ref = run_case(1, 4, 2, 1300, 1300, D, "bf16", VARIANTS[name], seed=13)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("S", [1, 2, 63, 64, 127, 128, 129, 200, 257, 511, 1025, 1100, 1537])
def test_lengths_causal(S):
    (o, lse), o_ref, l_ref = run_case(1, 2, 2, S, S, 128, "bf16", dict(mask=1), seed=S)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("Sq,Skv", [(100, 300), (300, 100), (1, 257), (257, 1), (129, 640)])
@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_sq_ne_skv(Sq, Skv, mask, D):
    (o, lse), o_ref, l_ref = run_case(1, 2, 1, Sq, Skv, D, "bf16", dict(mask=mask), seed=Sq + Skv)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (700, 64)])
@pytest.mark.parametrize("name", ["window", "causal_alibi", "softcap", "boost", "window_boost"])
@pytest.mark.parametrize("D,dtype", [(64, "f32"), (128, "bf16")])
def test_sq_ne_skv_modifiers(Sq, Skv, name, D, dtype):
    """Unequal lengths with every modifier and the window (absolute indices;
    with the window and Sq > Skv + window - 1 the last rows have no key)."""
    (o, lse), o_ref, l_ref = run_case(1, 4, 2, Sq, Skv, D, dtype, VARIANTS[name], seed=Sq * 3 + Skv)
    check_out(o, o_ref, dtype)
    check_lse(lse, l_ref)


# Local boost at the edges of its radius: 0 (no pair boosted, the unmodified
# scores), 1 (the diagonal only), and radii at and far past every |i - j|
# (all pairs boosted; 2^31 - 1 would overflow radius arithmetic done in int).
BOOST_EDGES = [0, 1, 699, 700 + 333, 2**31 - 1]


@pytest.mark.parametrize("radius", BOOST_EDGES)
@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("Sq,D,dtype", [(333, 128, "bf16"), (700, 64, "f32"), (1300, 128, "bf16")])
def test_boost_radius_edges(radius, mask, Sq, D, dtype):
    """Sq = 1300 takes the ping-pong kernel, the others the 4-wave kernel;
    keys 333 long except at Sq = 1300 (Skv = Sq)."""
    Skv = Sq if Sq == 1300 else 333
    spec = dict(mask=mask, mod=3, boost_radius=radius, boost_factor=2.0)
    (o, lse), o_ref, l_ref = run_case(1, 2, 1, Sq, Skv, D, dtype, spec, seed=radius % 1000 + Sq)
    check_out(o, o_ref, dtype)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (8, 2), (8, 1)])
@pytest.mark.parametrize("D,dtype", [(128, "bf16"), (64, "f32")])
def test_gqa_ratios(Hq, Hkv, D, dtype):
    (o, lse), o_ref, l_ref = run_case(2, Hq, Hkv, 260, 260, D, dtype, dict(mask=1, mod=1), seed=Hq * 10 + Hkv)
    check_out(o, o_ref, dtype)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("name", ["none", "causal", "window", "document", "document_alibi", "window_boost"])
def test_block_mask_path(name):
    """The block-mask path (lists of non-empty 128-blocks, FULL blocks skip
    the elementwise mask) matches the oracle."""
    (o, lse), o_ref, l_ref = run_case(2, 2, 2, 700, 700, 128, "bf16", VARIANTS[name], seed=5, block_mask=True)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("name", ["causal", "document", "window_boost"])
@pytest.mark.parametrize("D", [64, 128])
def test_block_mask_path_f32(name, D):
    """fp32 inputs through the block-mask path (fp32 products, 32-key steps)."""
    (o, lse), o_ref, l_ref = run_case(1, 2, 2, 450, 450, D, "f32", VARIANTS[name], seed=6, block_mask=True)
    check_out(o, o_ref, "f32")
    check_lse(lse, l_ref)


def test_lse_does_not_change_output():
    """Writing the LSE must not change O: same arithmetic, bit-identical."""
    q, k, v = (dev(t) for t in synth.qkv(2, 4, 2, 300, 300, 128, 3))
    for spec in (dict(mask=1), dict(mask=2, window=50, mod=2, softcap=30.0)):
        o1 = fa.forward(q, k, v, **spec)
        o2, _ = fa.forward(q, k, v, return_lse=True, **spec)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)


def test_deterministic():
    q, k, v = (dev(t) for t in synth.qkv(2, 4, 2, 640, 640, 128, 4))
    a, la = fa.forward(q, k, v, mask=1, mod=1, return_lse=True)
    b, lb = fa.forward(q, k, v, mask=1, mod=1, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_explicit_alibi_slopes():
    slopes = torch.tensor([0.5, 0.25, 0.125, 0.0], dtype=torch.float32)
    q, k, v = synth.qkv(1, 4, 4, 150, 150, 64, 9)
    o, lse = fa.forward(dev(q), dev(k), dev(v), mask=1, mod=1, alibi_slopes=dev(slopes), return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(q, k, v, f32_scale(64), oracle.Variant(mask=1, mod=1, slopes=slopes.numpy()))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


def test_zero_scale_uniform():
    """scale 0 gives uniform weights over the admissible keys."""
    q, k, v = synth.qkv(1, 2, 2, 200, 200, 64, 10)
    o, lse = fa.forward(dev(q), dev(k), dev(v), scale=0.0, mask=1, return_lse=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(q, k, v, 0.0, oracle.Variant(mask=1))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


def test_window_one_is_identity():
    q, k, v = synth.qkv(1, 2, 2, 300, 300, 128, 12)
    o = fa.forward(dev(q), dev(k), dev(v), mask=2, window=1)
    torch.cuda.synchronize()
    check_out(o, v.to(torch.float64).numpy(), "bf16")


def test_empty_inputs():
    """B = 0 and Sq = 0 are no-ops; Skv = 0 gives O = 0 and LSE = -inf."""
    z = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device="cuda")
    fa.forward(z, z, z)
    q = torch.randn(1, 2, 0, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(1, 2, 5, 64, device="cuda").to(torch.bfloat16)
    fa.forward(q, k, k)
    q = torch.randn(1, 2, 70, 64, device="cuda").to(torch.bfloat16)
    e = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    o, lse = fa.forward(q, e, e, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_rows_without_keys():
    """Causal with Sq > Skv never empties a row, but a document mask whose
    block list skips everything cannot happen either; the explicit empty-row
    case is Skv = 0 above.  Here: rows past Skv under causal still see keys."""
    (o, lse), o_ref, l_ref = run_case(1, 1, 1, 190, 60, 64, "bf16", dict(mask=1), seed=2)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


def test_visited_counts_analytic():
    """Key steps visited per 128-row query tile equal the number of
    kernel-width key tiles that hold at least one admissible pair."""
    B, H, S = 1, 2, 700
    step = fa.fa_fwd_kv_step(128, fa.FA_BF16)
    q, k, v = (dev(t) for t in synth.qkv(B, H, H, S, S, 128, 1))
    for spec in (dict(mask=0), dict(mask=1), dict(mask=2, window=200)):
        nq = -(-S // 128)
        vis = torch.zeros((B, H, nq), dtype=torch.int32, device="cuda")
        fa.forward(q, k, v, visited=vis, **spec)
        torch.cuda.synchronize()
        var = oracle.Variant(**spec)
        for qt in range(nq):
            rows = np.arange(qt * 128, min(S, qt * 128 + 128))
            ok = oracle.allowed(var, 0, rows, np.arange(S))
            want = sum(1 for kt in range(-(-S // step)) if ok[:, kt * step:(kt + 1) * step].any())
            assert int(vis[0, 0, qt]) == want, (spec, qt, int(vis[0, 0, qt]), want)


@pytest.mark.parametrize("spec", [dict(mask=2, window=2200), dict(mask=2, window=2100, mod=1)])
def test_long_window(spec):
    """Windows longer than 2048 keys take the 256-row ping-pong kernel (short
    windows the 128-row kernel): ragged length, several tiles per window."""
    (o, lse), o_ref, l_ref = run_case(1, 2, 1, 2600, 2600, 128, "bf16", spec, seed=31)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("mask", [0, 1])
def test_softcap_mixed_forms(mask):
    """Key blocks of alternating scale (x1, x8): in the x8 blocks most scores
    saturate the cap (|s| >> c), in the x1 blocks none do, so every row mixes
    steps far out on both tails of tanh with steps near its linear part."""
    B, H, S, D = 1, 4, 700, 128
    q, k, v = synth.qkv(B, H, H, S, S, D, 31)
    f = torch.where((torch.arange(S) // 64) % 2 == 0, 1.0, 8.0)[None, None, :, None]
    k = (k.float() * f).to(torch.bfloat16)
    spec = dict(mask=mask, mod=2, softcap=30.0)
    o, lse = fa.forward(dev(q), dev(k), dev(v), return_lse=True, **spec)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(q, k, v, f32_scale(D), oracle.Variant(**spec))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("B,Hq,Hkv,S", [(2, 8, 4, 700), (1, 16, 8, 1300), (4, 8, 2, 200), (2, 16, 8, 2600)])
def test_xcd_pinned_schedule(B, Hq, Hkv, S):
    """B * Hkv a multiple of 8 pins every (batch, kv-head) unit to one XCD,
    one to four units and one to four query heads per unit on each, at 1 to
    21 tiles per head (128- and 256-row tiles): every tile of every head must
    be computed exactly once."""
    (o, lse), o_ref, l_ref = run_case(B, Hq, Hkv, S, S, 128, "bf16", dict(mask=1), seed=B * S)
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("S,rows", [(700, 128), (2600, 256)])
def test_wg_trace_records(S, rows):
    """fa_mask_params.wg_trace: one record per query tile of the static
    schedule (128-row tiles up to 1024 keys, 256-row ping-pong tiles above),
    end after start, the causal key-step count of each tile, an XCD id below
    8; the output is the same bits as without the trace."""
    B, Hq, Hkv, D = 2, 4, 2, 128
    q, k, v = (dev(t) for t in synth.qkv(B, Hq, Hkv, S, S, D, 77))
    o_ref = fa.forward(q, k, v, mask=1)
    tr = fa.new_wg_trace(B, Hq, S)
    o = fa.forward(q, k, v, mask=1, wg_trace=tr)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
    recs = fa.decode_wg_trace(tr.cpu().numpy())
    n_tiles = B * Hq * -(-S // rows)
    assert sorted(r["P"] for r in recs) == list(range(n_tiles))
    steps_of_tile = {}
    for t in range(-(-S // rows)):
        steps_of_tile[t] = -(-min(S, (t + 1) * rows) // 64)
    for r in recs:
        assert r["end_us"] > r["start_us"] and r["rows"] == rows and 0 <= r["xcd"] < 8
        assert r["steps"] in steps_of_tile.values()
    assert sorted(r["steps"] for r in recs) == sorted(list(steps_of_tile.values()) * B * Hq)
