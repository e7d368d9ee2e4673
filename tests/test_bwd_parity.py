"""Backward pass: HIP library against the fp64 oracle's chain-rule gradients."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.floors import backward_floors, rounding_mean
from tests.gpu_util import check_out, dev, f32_scale
from tests.test_fwd_parity import VARIANTS, doc_ids_for

pytestmark = pytest.mark.gpu


def run_bwd(B, Hq, Hkv, S, D, spec, seed, block_mask=False):
    q, k, v = synth.qkv(B, Hq, Hkv, S, S, D, seed)
    do = synth.randn((B, Hq, S, D), seed + 100)
    scale = f32_scale(D)
    doc = doc_ids_for(B, S, seed) if spec.get("mask") == 3 else None
    var = oracle.Variant(doc_ids=None if doc is None else doc.numpy(), **spec)
    bm = None
    if block_mask:
        bm = fa.build_block_mask(spec.get("mask", 0), B, S, S, window=spec.get("window", 0), doc_ids=dev(doc))
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(qd, kd, vd, scale=scale, doc_ids=dev(doc), return_lse=True, block_mask=bm, **spec)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, scale=scale, doc_ids=dev(doc), block_mask=bm, **spec)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(q, k, v, do, scale, var)
    return (dq, dk, dv), (rq, rk, rv)


# Non-causal ALiBi with slopes 2^-2, 2^-4, ... sends every query to the last
# keys, so dK of those keys sums ~333 large terms (|dK| ~ 10).  Rounding only
# the dS operand of that contraction to bf16 (everything else exact, fp64 on
# the CPU) already leaves 1.67e-2 (D=64) / 1.64e-2 (D=128) of error beyond the
# output's own rounding: the floor of any bf16-operand backward, with no room
# under 2e-2 for the fp32 accumulation (tests/test_bwd_floor.py).  This case
# gets 3e-2.
MAX_EXCESS = {"none_alibi": 3e-2}
# The same holds, more strongly, when 700 causal queries reach 64 keys under
# ALiBi (every row of head 0 weighs the last keys; |dK| ~ 12, |dV| ~ 24):
# rounding dS alone leaves 2.04e-2 (D=64) / 1.58e-2 (D=128) on dK, rounding P
# alone 2.21e-2 / 2.92e-2 on dV (tests/test_bwd_floor.py).  That case gets
# 4e-2, and its means are taken beyond the outputs' own rounding, which alone
# averages 1.3e-3 at these magnitudes.
MAX_EXCESS_LENGTHS = {(700, 64, "causal_alibi"): 4e-2}


@pytest.mark.parametrize("name", sorted(VARIANTS))
@pytest.mark.parametrize("D", [64, 128])
def test_variants(name, D):
    got, ref = run_bwd(1, 4, 2, 333, D, VARIANTS[name], seed=21)
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what, max_excess=MAX_EXCESS.get(name))


@pytest.mark.parametrize("radius", [0, 1, 333, 2**31 - 1])
@pytest.mark.parametrize("mask", [0, 1])
def test_boost_radius_edges(radius, mask):
    """Local boost with radius 0 (no pair boosted), 1 (the diagonal only) and
    radii covering every pair, the last past int arithmetic on the radius."""
    spec = dict(mask=mask, mod=3, boost_radius=radius, boost_factor=2.0)
    seed = radius % 1000 + 5
    got, ref = run_bwd(1, 2, 1, 333, 128, spec, seed=seed)
    # A factor of 2 on every pair doubles the effective scale, and the bf16
    # operands alone then leave up to ~3e-2 on dQ / dK (causal): such cases
    # are held to 1.5x their floor, as the seeded random cases are.
    q, k, v = synth.qkv(1, 2, 1, 333, 333, 128, seed)
    floors = backward_floors(q, k, v, synth.randn((1, 2, 333, 128), seed + 100), f32_scale(128),
                             oracle.Variant(**spec))
    for g, r, what, fl in zip(got, ref, ("dQ", "dK", "dV"), floors):
        check_out(g, r, "bf16", f"{what} floor {fl:.2e}", max_excess=max(2e-2, 1.5 * fl),
                  rounding_mean=rounding_mean(r) > 1e-3)


@pytest.mark.parametrize("S", [1, 64, 127, 129, 260])
def test_lengths_causal(S):
    got, ref = run_bwd(1, 2, 2, S, 128, dict(mask=1), seed=S + 3)
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (4, 1)])
@pytest.mark.parametrize("D", [64, 128])
def test_gqa_group_sums(Hq, Hkv, D):
    got, ref = run_bwd(2, Hq, Hkv, 200, D, dict(mask=1, mod=1), seed=7)
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)


@pytest.mark.parametrize("name", ["causal", "document", "window_boost", "none"])
def test_block_mask_path(name):
    got, ref = run_bwd(1, 2, 2, 600, 128, VARIANTS[name], seed=8, block_mask=True)
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)


def test_deterministic():
    q, k, v = (dev(t) for t in synth.qkv(1, 4, 2, 400, 400, 128, 30))
    do = dev(synth.randn((1, 4, 400, 128), 31))
    o, lse = fa.forward(q, k, v, mask=1, return_lse=True)
    a = fa.backward(q, k, v, o, do, lse, mask=1)
    b = fa.backward(q, k, v, o, do, lse, mask=1)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_empty_queries_zero_key_grads():
    """Sq = 0: no query sees any key, so dK = dV = 0."""
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn(1, 2, 50, 64, device="cuda").to(torch.bfloat16)
    dk = torch.full_like(k, 7.0)
    dv = torch.full_like(k, 7.0)
    fa.backward(q, k, k, q, q, torch.empty((1, 2, 0), device="cuda"), grads=(q, dk, dv))
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)


LENGTH_SPECS = {"none": dict(mask=0), "causal": dict(mask=1), "causal_alibi": dict(mask=1, mod=1),
                "window": dict(mask=2, window=90)}


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (64, 700), (700, 64)])
@pytest.mark.parametrize("name", sorted(LENGTH_SPECS))
@pytest.mark.parametrize("D", [64, 128])
def test_sq_ne_skv(Sq, Skv, name, D):
    """Query and key lengths differ (absolute indices: causal is j <= i).
    With the window and Sq > Skv + window - 1 the last rows have no key at
    all (O = 0, LSE = -inf): their gradients are zero."""
    spec = LENGTH_SPECS[name]
    q, _, _ = synth.qkv(1, 4, 2, Sq, Sq, D, 40)
    _, k, v = synth.qkv(1, 4, 2, Skv, Skv, D, 41)
    do = synth.randn((1, 4, Sq, D), 42)
    scale = f32_scale(D)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(qd, kd, vd, scale=scale, return_lse=True, **spec)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, scale=scale, **spec)
    torch.cuda.synchronize()
    rq, rk, rv = oracle.backward(q, k, v, do, scale, oracle.Variant(**spec))
    for g, r, what in zip((dq, dk, dv), (rq, rk, rv), ("dQ", "dK", "dV")):
        bar = MAX_EXCESS_LENGTHS.get((Sq, Skv, name))
        check_out(g, r, "bf16", what, max_excess=bar, rounding_mean=bar is not None)


@pytest.mark.parametrize("Sq,Skv", [(300, 520), (520, 300)])
@pytest.mark.parametrize("name", ["none", "causal", "window"])
@pytest.mark.parametrize("D", [64, 128])
def test_block_mask_unequal_lengths(Sq, Skv, name, D):
    """Forward and backward through a block mask built for Sq != Skv, GQA."""
    spec = LENGTH_SPECS[name]
    q, _, _ = synth.qkv(1, 4, 2, Sq, Sq, D, 50)
    _, k, v = synth.qkv(1, 4, 2, Skv, Skv, D, 51)
    do = synth.randn((1, 4, Sq, D), 52)
    scale = f32_scale(D)
    bm = fa.build_block_mask(spec["mask"], 1, Sq, Skv, window=spec.get("window", 0))
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(qd, kd, vd, scale=scale, return_lse=True, block_mask=bm, **spec)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, scale=scale, block_mask=bm, **spec)
    torch.cuda.synchronize()
    var = oracle.Variant(**spec)
    o_ref, _ = oracle.forward(q, k, v, scale, var)
    rq, rk, rv = oracle.backward(q, k, v, do, scale, var)
    check_out(o, o_ref, "bf16", "O")
    for g, r, what in zip((dq, dk, dv), (rq, rk, rv), ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)


def test_phases_on_two_streams():
    """DELTA, then DK/DV and DQ on two streams (each waiting for DELTA by an
    event), gives the same bits as the single fa_bwd call."""
    B, Hq, Hkv, S, D = 1, 4, 2, 700, 128
    q, k, v = (dev(t) for t in synth.qkv(B, Hq, Hkv, S, S, D, 70))
    do = dev(synth.randn((B, Hq, S, D), 71))
    spec = dict(mask=fa.MASK_CAUSAL, mod=fa.MOD_ALIBI)
    o, lse = fa.forward(q, k, v, return_lse=True, **spec)
    ref = fa.backward(q, k, v, o, do, lse, **spec)
    ws = torch.empty(fa.fa_bwd_workspace_bytes(B, Hq, S, D), dtype=torch.uint8, device="cuda")
    grads = (torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(v, float("nan")))
    main = torch.cuda.current_stream()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    fa.backward(q, k, v, o, do, lse, workspace=ws, grads=grads, phases=fa.FA_BWD_DELTA, stream=main, **spec)
    s1.wait_stream(main)
    s2.wait_stream(main)
    fa.backward(q, k, v, o, do, lse, workspace=ws, grads=grads, phases=fa.FA_BWD_DKDV, stream=s1, **spec)
    fa.backward(q, k, v, o, do, lse, workspace=ws, grads=grads, phases=fa.FA_BWD_DQ, stream=s2, **spec)
    main.wait_stream(s1)
    main.wait_stream(s2)
    torch.cuda.synchronize()
    for got, want, what in zip(grads, ref, ("dQ", "dK", "dV")):
        assert torch.equal(got, want), what


FUSED_CASES = [
    # (B, Hq, Hkv, Sq, Skv, D, spec, block mask)
    (1, 4, 2, 333, 333, 64, dict(mask=fa.MASK_CAUSAL), False),
    (2, 4, 4, 700, 700, 128, dict(mask=fa.MASK_NONE, mod=fa.MOD_SOFTCAP, softcap=30.0), False),
    (1, 4, 2, 333, 500, 128, dict(mask=fa.MASK_CAUSAL, mod=fa.MOD_ALIBI), False),
    (2, 2, 1, 900, 900, 128, dict(mask=fa.MASK_DOCUMENT), True),
    (1, 2, 2, 450, 450, 64, dict(mask=fa.MASK_SLIDING_WINDOW, window=100, mod=fa.MOD_LOCAL_BOOST, boost_radius=40,
                                boost_factor=1.1), True),
]


@pytest.mark.parametrize("case", FUSED_CASES, ids=[f"D{c[5]}-S{c[3]}x{c[4]}-m{c[6]['mask']}-bm{int(c[7])}"
                                                   for c in FUSED_CASES])
def test_fused_row_pass_same_bits(case):
    """A call holding DELTA and DQ runs one launch, the dQ kernel doing the
    row pass for its own rows.  Its row arrays (rowsum(dO * O), LSE in log2
    units) and all three gradients must equal, bit for bit, those of the row
    pass and the kernels launched one by one, for every split of the phases."""
    B, Hq, Hkv, Sq, Skv, D, spec, use_bm = case
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, 80 + Sq)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, 81 + Skv)
    q, k, v = dev(q), dev(k), dev(v)
    do = dev(synth.randn((B, Hq, Sq, D), 82))
    doc = dev(doc_ids_for(B, Sq, 83)) if spec["mask"] == fa.MASK_DOCUMENT else None
    bm = None
    if use_bm:
        bm = fa.build_block_mask(spec["mask"], B, Sq, Skv, window=spec.get("window", 0), doc_ids=doc)
    kw = dict(doc_ids=doc, block_mask=bm, **spec)
    o, lse = fa.forward(q, k, v, return_lse=True, **kw)
    ws_bytes = fa.fa_bwd_workspace_bytes(B, Hq, Sq, D)

    def run(splits):
        ws = torch.full((ws_bytes,), 0xFF, dtype=torch.uint8, device="cuda")
        grads = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
        for ph in splits:
            fa.backward(q, k, v, o, do, lse, workspace=ws, grads=grads, phases=ph, **kw)
        torch.cuda.synchronize()
        return ws, grads

    one_by_one = run([fa.FA_BWD_DELTA, fa.FA_BWD_DKDV, fa.FA_BWD_DQ])
    rows_then_kv = run([fa.FA_BWD_DELTA | fa.FA_BWD_DQ, fa.FA_BWD_DKDV])
    all_in_one = run([fa.FA_BWD_DELTA | fa.FA_BWD_DKDV | fa.FA_BWD_DQ])
    n = B * Hq * Sq
    half = (n * 4 + 255) // 256 * 256
    ref_rows = [one_by_one[0][:n * 4].view(torch.float32), one_by_one[0][half:half + n * 4].view(torch.float32)]
    for got, label in ((rows_then_kv, "DELTA|DQ, DKDV"), (all_in_one, "fa_bwd")):
        assert torch.equal(got[0][:n * 4], one_by_one[0][:n * 4]), (label, "rowsum(dO * O)")
        assert torch.equal(got[0][half:half + n * 4], one_by_one[0][half:half + n * 4]), (label, "LSE log2")
        for g, r, what in zip(got[1], one_by_one[1], ("dQ", "dK", "dV")):
            assert torch.equal(g, r), (label, what)
    # The row pass itself against its definition on the rounded O (fp64 here).
    want = (do.double() * o.double()).sum(-1).reshape(-1)
    assert torch.allclose(ref_rows[0].double(), want, rtol=1e-5, atol=1e-5)
    assert not torch.isnan(ref_rows[1]).any()


@pytest.mark.parametrize("Sq,Skv", [(700, 700), (333, 500), (1500, 1500)])
def test_huge_window_is_causal(Sq, Skv):
    """A window of 2^31 - 1 keys admits exactly the causal pairs: forward and
    backward give the causal mask's bits (the host clamps the window to
    max(Sq, Skv), so no kernel's range arithmetic overflows)."""
    B, Hq, Hkv, D = 1, 4, 2, 128
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, 60 + Sq)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, 61 + Skv)
    q, k, v = dev(q), dev(k), dev(v)
    do = dev(synth.randn((B, Hq, Sq, D), 62))
    res = []
    for spec in (dict(mask=fa.MASK_CAUSAL), dict(mask=fa.MASK_SLIDING_WINDOW, window=2**31 - 1)):
        o, lse = fa.forward(q, k, v, return_lse=True, **spec)
        res.append((o, lse, *fa.backward(q, k, v, o, do, lse, **spec)))
    torch.cuda.synchronize()
    for a, b, what in zip(res[0], res[1], ("O", "LSE", "dQ", "dK", "dV")):
        assert torch.equal(a, b), what


@pytest.mark.parametrize("B,Hq,Hkv,S", [(2, 8, 4, 700), (4, 8, 2, 200)])
def test_xcd_pinned_schedule(B, Hq, Hkv, S):
    """dQ and dK/dV under the XCD-pinned schedule (B * Hkv a multiple of 8),
    with GQA groups of 2 and 4 query heads."""
    got, ref = run_bwd(B, Hq, Hkv, S, 128, dict(mask=1), seed=B * S + 1)
    for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)


def test_wg_trace_records():
    """fa_mask_params.wg_trace in the backward: one record per dK/dV
    workgroup (key tiles), then one per dQ workgroup, each with its query
    or key step count; the gradients are the same bits as without it."""
    B, Hq, Hkv, S, D = 2, 4, 2, 700, 128
    q, k, v = (dev(t) for t in synth.qkv(B, Hq, Hkv, S, S, D, 78))
    do = dev(synth.randn((B, Hq, S, D), 79))
    o, lse = fa.forward(q, k, v, mask=1, return_lse=True)
    ref = fa.backward(q, k, v, o, do, lse, mask=1)
    tr = fa.new_wg_trace(B, Hq, S, Hkv=Hkv, Skv=S)
    got = fa.backward(q, k, v, o, do, lse, mask=1, wg_trace=tr)
    torch.cuda.synchronize()
    for x, y in zip(got, ref):
        assert torch.equal(x, y)
    rec = tr.cpu().numpy()
    n_t = -(-S // 128)
    n_kv = B * Hkv * n_t
    kv = fa.decode_wg_trace(rec[:n_kv])
    dq = fa.decode_wg_trace(rec[n_kv:])
    assert sorted(r["P"] for r in kv) == list(range(n_kv))
    assert sorted(r["P"] for r in dq) == list(range(B * Hq * n_t))
    # Causal: key tile kt visits the 32-row query steps from 4 kt on, for
    # each of the G = 2 query heads; query tile qt the 64-key steps up to it.
    n_qs = -(-S // 32)
    want_kv = sorted([2 * (n_qs - 4 * t) for t in range(n_t)] * (B * Hkv))
    want_dq = sorted([-(-min(S, 128 * (t + 1)) // 64) for t in range(n_t)] * (B * Hq))
    assert sorted(r["steps"] for r in kv) == want_kv
    assert sorted(r["steps"] for r in dq) == want_dq
    assert all(r["end_us"] > r["start_us"] and 0 <= r["xcd"] < 8 for r in kv + dq)
