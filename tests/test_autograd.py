"""fa.attention(): the library's forward and backward as one differentiable
torch operation.  It only marshals arguments, so its output and gradients
must be the direct calls' bits (fa.forward, then fa.backward with the
forward's O and LSE), and one case is checked end to end against the oracle."""
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import check_out, dev, f32_scale
from tests.test_fwd_parity import doc_ids_for

pytestmark = pytest.mark.gpu

CASES = [
    # (B, Hq, Hkv, S, D, spec, block mask)
    (2, 4, 2, 700, 128, dict(mask=fa.MASK_CAUSAL), False),
    (1, 4, 1, 333, 64, dict(mask=fa.MASK_NONE, mod=fa.MOD_ALIBI), False),
    (1, 2, 2, 900, 128, dict(mask=fa.MASK_DOCUMENT), True),
    (1, 2, 2, 500, 128, dict(mask=fa.MASK_SLIDING_WINDOW, window=64, mod=fa.MOD_SOFTCAP, softcap=30.0), False),
]


def _leaf(t):
    return dev(t).detach().requires_grad_(True)


@pytest.mark.parametrize("case", CASES, ids=[f"m{c[5]['mask']}-D{c[4]}-bm{int(c[6])}" for c in CASES])
def test_same_bits_as_direct_calls(case):
    B, Hq, Hkv, S, D, spec, use_bm = case
    q0, k0, v0 = synth.qkv(B, Hq, Hkv, S, S, D, 90 + S)
    do = dev(synth.randn((B, Hq, S, D), 91))
    doc = dev(doc_ids_for(B, S, 92)) if spec["mask"] == fa.MASK_DOCUMENT else None
    bm = fa.build_block_mask(spec["mask"], B, S, S, window=spec.get("window", 0), doc_ids=doc) if use_bm else None
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    o = fa.attention(q, k, v, doc_ids=doc, block_mask=bm, **spec)
    o.backward(do)
    torch.cuda.synchronize()
    qd, kd, vd = dev(q0), dev(k0), dev(v0)
    o_ref, lse = fa.forward(qd, kd, vd, doc_ids=doc, block_mask=bm, return_lse=True, **spec)
    g_ref = fa.backward(qd, kd, vd, o_ref, do, lse, doc_ids=doc, block_mask=bm, **spec)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    for g, r, what in zip((q.grad, k.grad, v.grad), g_ref, ("dQ", "dK", "dV")):
        assert torch.equal(g, r), what


def test_relative_bias_table_gradient():
    B, Hq, Hkv, S, D = 1, 2, 2, 400, 128
    q0, k0, v0 = synth.qkv(B, Hq, Hkv, S, S, D, 93)
    table = dev(0.5 * synth.randn((Hq, 2 * S - 1), 94).float())
    do = dev(synth.randn((B, Hq, S, D), 95))
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    t = table.detach().clone().requires_grad_(True)
    o = fa.attention(q, k, v, mask=fa.MASK_CAUSAL, mod=fa.MOD_REL_BIAS, rel_bias=t)
    o.backward(do)
    qd, kd, vd = dev(q0), dev(k0), dev(v0)
    o_ref, lse = fa.forward(qd, kd, vd, mask=fa.MASK_CAUSAL, mod=fa.MOD_REL_BIAS, rel_bias=table, return_lse=True)
    ref = fa.backward(qd, kd, vd, o_ref, do, lse, mask=fa.MASK_CAUSAL, mod=fa.MOD_REL_BIAS, rel_bias=table,
                      rel_bias_grad=True)
    torch.cuda.synchronize()
    for g, r, what in zip((q.grad, k.grad, v.grad, t.grad), ref, ("dQ", "dK", "dV", "table")):
        assert torch.equal(g, r), what


def test_noncontiguous_upstream_gradient_and_oracle():
    """A loss whose gradient reaches O as a transposed view, checked against
    the oracle's chain rule (the binding makes the upstream gradient dense)."""
    B, Hq, Hkv, S, D = 1, 2, 1, 300, 64
    q0, k0, v0 = synth.qkv(B, Hq, Hkv, S, S, D, 96)
    w = dev(synth.randn((B, Hq, D, S), 97))  # weights laid out [.., D, S]
    q, k, v = _leaf(q0), _leaf(k0), _leaf(v0)
    o = fa.attention(q, k, v, mask=fa.MASK_CAUSAL)
    (o.float() * w.float().transpose(-1, -2)).sum().backward()
    do = w.transpose(-1, -2).contiguous()
    rq, rk, rv = oracle.backward(q0, k0, v0, do.cpu(), f32_scale(D), oracle.Variant(mask=fa.MASK_CAUSAL))
    for g, r, what in zip((q.grad, k.grad, v.grad), (rq, rk, rv), ("dQ", "dK", "dV")):
        check_out(g, r, "bf16", what)
