"""Learnable relative-position bias: forward, backward and the table gradient
of the HIP library against the fp64 oracle.

The modifier adds table[h][i - j + Skv - 1] to the scaled score (the
FlexAttention/FA4 page names gradients of learnable bias tensors among
FlexAttention's limits, "섹션별 상세").  The table gradient is the sum of dS'
over every (batch, query, key) pair on a diagonal, and is checked against
the oracle with a bound that scales with the absolute sum of those terms.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import check_lse, check_out, dev, f32_scale
from tests.test_fwd_parity import doc_ids_for

pytestmark = pytest.mark.gpu

MASKS = {"none": dict(mask=0), "causal": dict(mask=1), "window": dict(mask=2, window=90), "document": dict(mask=3)}

# Table gradient bar.  Each dS'_ij = p_ij (dP_ij - delta_i) is formed in
# fp32, but delta_i = rowsum(dO_i * O_i) comes from the forward's bf16
# output, whose error is at most half a bf16 ulp plus the effect of the
# bf16-rounded probabilities in the P V product:
#   |delta_i error| <= 2^-9 sum_d |dO_id| (|O_id| + sum_j p_ij |V_jd|) =: eps_i,
# and eps_i enters every term of row i with weight p_ij.  Per table entry r:
#   |err_r| <= 2 sum_(i,j on r) p_ij eps_i + 1e-3 sum_(i,j on r) |dS'_ij| + 1e-6
# (factor 2 of margin; the second term covers the fp32 exp2 and sums).  A
# numpy model of exactly these roundings, fp64 otherwise, reaches 0.03 of
# this bound on the test shapes.
GRAD_REL, GRAD_ABS = 1e-3, 1e-6


def _variant(spec, doc, table, Skv):
    return oracle.Variant(doc_ids=None if doc is None else doc.numpy(), mod=oracle.MOD_REL_BIAS,
                          rel_bias=table.numpy(), rel_origin=Skv - 1, **spec)


def _error_scales(q, k, v, do, scale, var):
    """Per table entry: sum |dS'| and sum p_ij eps_i."""
    q, k, v, do = (oracle.attention._f64(t) for t in (q, k, v, do))
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    A = np.zeros((Hq, Sq + Skv - 1))
    E = np.zeros((Hq, Sq + Skv - 1))
    idx = oracle.attention.rel_index(var, np.arange(Sq), np.arange(Skv))
    for b in range(B):
        for h in range(Hq):
            hk = oracle.attention.kv_head(h, Hq, Hkv)
            _, _, _, O, _, dsp = oracle.attention.backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, var,
                                                                b, h, Hq, with_dsp=True)
            P = oracle.probabilities(q[b, h], k[b, hk], scale, var, b, h, Hq)
            eps = 2.0 ** -9 * np.sum(np.abs(do[b, h]) * (np.abs(O) + P @ np.abs(v[b, hk])), axis=1)
            np.add.at(A[h], idx, np.abs(dsp))
            np.add.at(E[h], idx, P * eps[:, None])
    return A, E


def check_grad(got, ref, scales, what="rel_bias_grad"):
    A, E = scales
    g = got.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g))
    err = np.abs(g - ref)
    bound = 2.0 * E + GRAD_REL * A + GRAD_ABS
    worst = float(np.max(err / bound, initial=0.0))
    assert worst <= 1.0, f"{what}: worst |err| / bound = {worst:.3f}, max err {err.max():.3e}"


def run(B, Hq, Hkv, Sq, Skv, D, spec, seed, dtype="bf16", block_mask=False, std=1.0):
    q, k, v = synth.qkv(B, Hq, Hkv, Sq, Skv, D, seed, dtype)
    table = synth.rel_bias_table(Hq, Sq, Skv, seed + 50, std)
    doc = doc_ids_for(B, Sq, seed) if spec.get("mask") == 3 else None
    bm = None
    if block_mask:
        bm = fa.build_block_mask(spec.get("mask", 0), B, Sq, Skv, window=spec.get("window", 0), doc_ids=dev(doc))
    scale = f32_scale(D)
    o, lse = fa.forward(dev(q), dev(k), dev(v), scale=scale, doc_ids=dev(doc), mod=fa.MOD_REL_BIAS,
                        rel_bias=dev(table), block_mask=bm, return_lse=True, **spec)
    torch.cuda.synchronize()
    return (q, k, v, table, doc, bm, scale), (o, lse)


@pytest.mark.parametrize("name", sorted(MASKS))
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_forward(name, D, dtype):
    (q, k, v, table, doc, _, scale), (o, lse) = run(2, 4, 2, 333, 333, D, MASKS[name], 61, dtype)
    o_ref, l_ref = oracle.forward(q, k, v, scale, _variant(MASKS[name], doc, table, 333))
    check_out(o, o_ref, dtype)
    check_lse(lse, l_ref)


@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_forward_ping_pong_sizes(mask, D):
    """Past 1024 keys the unmasked and causal forwards take the ping-pong
    kernel, whose bias slices are loaded by the group that issues no tiles."""
    (q, k, v, table, doc, _, scale), (o, lse) = run(1, 4, 2, 1300, 1300, D, dict(mask=mask), 63)
    o_ref, l_ref = oracle.forward(q, k, v, scale, _variant(dict(mask=mask), doc, table, 1300))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("Sq,Skv", [(100, 300), (300, 100), (1, 257), (257, 1)])
@pytest.mark.parametrize("mask", [0, 1])
def test_forward_sq_ne_skv(Sq, Skv, mask):
    (q, k, v, table, doc, _, scale), (o, lse) = run(1, 2, 1, Sq, Skv, 128, dict(mask=mask), Sq + 3 * Skv)
    o_ref, l_ref = oracle.forward(q, k, v, scale, _variant(dict(mask=mask), doc, table, Skv))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("name", ["causal", "document", "window"])
def test_forward_block_mask(name):
    (q, k, v, table, doc, _, scale), (o, lse) = run(2, 2, 2, 700, 700, 128, MASKS[name], 62, block_mask=True)
    o_ref, l_ref = oracle.forward(q, k, v, scale, _variant(MASKS[name], doc, table, 700))
    check_out(o, o_ref, "bf16")
    check_lse(lse, l_ref)


def _backward_case(B, Hq, Hkv, Sq, Skv, D, spec, seed, block_mask=False):
    (q, k, v, table, doc, bm, scale), (o, lse) = run(B, Hq, Hkv, Sq, Skv, D, spec, seed, block_mask=block_mask)
    do = synth.randn((B, Hq, Sq, D), seed + 100)
    dq, dk, dv, gt = fa.backward(dev(q), dev(k), dev(v), o, dev(do), lse, scale=scale, doc_ids=dev(doc),
                                 mod=fa.MOD_REL_BIAS, rel_bias=dev(table), rel_bias_grad=True, block_mask=bm,
                                 **spec)
    torch.cuda.synchronize()
    var = _variant(spec, doc, table, Skv)
    rq, rk, rv = oracle.backward(q, k, v, do, scale, var)
    for g, r, what in zip((dq, dk, dv), (rq, rk, rv), ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what, rounding_mean=Skv == 1 and what == "dV")
    check_grad(gt, oracle.rel_bias_grad(q, k, v, do, scale, var), _error_scales(q, k, v, do, scale, var))


@pytest.mark.parametrize("name", sorted(MASKS))
@pytest.mark.parametrize("D", [64, 128])
def test_backward(name, D):
    _backward_case(2, 4, 2, 333, 333, D, MASKS[name], 63)


@pytest.mark.parametrize("Sq,Skv", [(200, 330), (330, 200), (1, 130), (130, 1)])
def test_backward_sq_ne_skv(Sq, Skv):
    _backward_case(1, 2, 2, Sq, Skv, 128, dict(mask=0), 64)


@pytest.mark.parametrize("name", ["causal", "document"])
def test_backward_block_mask(name):
    _backward_case(1, 2, 1, 600, 600, 128, MASKS[name], 65, block_mask=True)


def test_gradient_deterministic_and_phase_split():
    """The table gradient is bit-identical across runs, and the DQ phase alone
    (after DELTA) produces it."""
    (q, k, v, table, _, _, scale), (o, lse) = run(1, 2, 2, 400, 400, 128, dict(mask=1), 66)
    do = dev(synth.randn((1, 2, 400, 128), 166))
    args = (dev(q), dev(k), dev(v), o, do, lse)
    kw = dict(scale=scale, mask=1, mod=fa.MOD_REL_BIAS, rel_bias=dev(table), rel_bias_grad=True)
    g1 = fa.backward(*args, **kw)[3]
    g2 = fa.backward(*args, **kw)[3]
    ws = torch.empty(fa.fa_bwd_workspace_bytes(1, 2, 400, 128), dtype=torch.uint8, device="cuda")
    fa.backward(*args, workspace=ws, phases=fa.FA_BWD_DELTA, **kw)
    g3 = fa.backward(*args, workspace=ws, phases=fa.FA_BWD_DQ, **kw)[3]
    torch.cuda.synchronize()
    assert torch.equal(g1, g2) and torch.equal(g1, g3)


def test_zero_table_equals_no_modifier():
    """An all-zero table gives the unmodified forward and backward (same
    probabilities; the gradient still comes out)."""
    q, k, v = (dev(t) for t in synth.qkv(1, 2, 2, 300, 300, 64, 67))
    do = dev(synth.randn((1, 2, 300, 64), 167))
    zero = torch.zeros((2, 599), dtype=torch.float32, device="cuda")
    o0, l0 = fa.forward(q, k, v, mask=1, return_lse=True)
    o1, l1 = fa.forward(q, k, v, mask=1, mod=fa.MOD_REL_BIAS, rel_bias=zero, return_lse=True)
    g0 = fa.backward(q, k, v, o0, do, l0, mask=1)
    g1 = fa.backward(q, k, v, o1, do, l1, mask=1, mod=fa.MOD_REL_BIAS, rel_bias=zero, rel_bias_grad=True)
    torch.cuda.synchronize()
    # at most one bf16 step apart (the exp arguments differ by fp32 rounding)
    a, b = o0.float(), o1.float()
    assert bool(torch.all((a - b).abs() <= 2 ** -7 * torch.maximum(a.abs(), b.abs()) + 1e-30))
    assert float((l0 - l1).abs().max()) <= 1e-5
    for a, b in zip(g0, g1[:3]):
        assert float((a.float() - b.float()).abs().max()) <= 2e-2


def test_empty_rows_zero_gradient():
    """Sq = 0: the table gradient is written and is zero."""
    q = torch.empty((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    k = torch.randn(1, 2, 50, 64, device="cuda").to(torch.bfloat16)
    table = torch.randn(2, 49, device="cuda")
    grad = torch.full((2, 49), 7.0, device="cuda")
    fa.backward(q, k, k, q, q, torch.empty((1, 2, 0), device="cuda"), mod=fa.MOD_REL_BIAS, rel_bias=table,
                rel_bias_grad=grad)
    torch.cuda.synchronize()
    assert torch.all(grad == 0)
