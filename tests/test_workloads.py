"""The benchmark workloads at full size, in the launch configuration bench.py
times, against the oracle.

Rows are independent given all keys, so each sampled query row is an exact
check: every (batch, head) is checked on >= 512 seeded rows that include the
first and last 128 rows and rows around tile, window and document edges.
The tiny fp32 workload is checked in full.  The backward pass of the causal
S=8192 workload is checked in full on two whole heads.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import check_lse, check_out, f32_scale

pytestmark = pytest.mark.gpu


def _variant(w, extras):
    doc = extras.get("doc_ids")
    return oracle.Variant(mask=w.mask, window=w.window, mod=w.mod, softcap=w.softcap,
                          boost_radius=w.boost_radius, boost_factor=w.boost_factor,
                          doc_ids=None if doc is None else doc.numpy())


def _run(w):
    q, k, v, extras = synth.workload_inputs(w)
    dev = "cuda"
    doc = extras["doc_ids"].to(dev) if "doc_ids" in extras else None
    bm = fa.build_block_mask(w.mask, w.B, w.S, w.S, doc_ids=doc) if w.mask == fa.MASK_DOCUMENT else None
    o, lse = fa.forward(q.to(dev), k.to(dev), v.to(dev), mask=w.mask, window=w.window, doc_ids=doc, mod=w.mod,
                        softcap=w.softcap, boost_radius=w.boost_radius, boost_factor=w.boost_factor,
                        block_mask=bm, return_lse=True)
    torch.cuda.synchronize()
    return q, k, v, extras, o.cpu(), lse.cpu()


def _edges(w, extras):
    e = [128 * t for t in range(1, w.S // 128)][::7]
    if w.window:
        e += [w.window, w.window + 128, 3 * w.window]
    if "doc_lengths" in extras:
        e += list(np.cumsum(extras["doc_lengths"])[:-1])
    return e


def test_tiny_mha_f32_full():
    w = synth.WORKLOADS["tiny_mha_f32"]
    q, k, v, extras, o, lse = _run(w)
    o_ref, l_ref = oracle.forward(q, k, v, f32_scale(w.D), _variant(w, extras))
    check_out(o, o_ref, "f32")
    check_lse(lse, l_ref)


@pytest.mark.parametrize("name", ["causal_prefill", "gqa_alibi", "gqa_softcap", "gqa_window", "gqa_boost",
                                  "gqa_causal", "doc_packed", "causal_fwd_bwd"])
def test_forward_sampled_rows(name):
    w = synth.WORKLOADS[name]
    q, k, v, extras, o, lse = _run(w)
    rows = synth.sample_rows(w.S, 512, w.seed + 7, extra=_edges(w, extras))
    o_ref, l_ref = oracle.forward(q, k, v, f32_scale(w.D), _variant(w, extras), rows=rows)
    check_out(o[:, :, rows], o_ref, "bf16")
    check_lse(lse[:, :, rows], l_ref)


def test_causal_backward_two_whole_heads():
    w = synth.WORKLOADS["causal_fwd_bwd"]
    q, k, v, extras = synth.workload_inputs(w)
    do = extras["do"]
    qd, kd, vd, dod = (t.to("cuda") for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, mask=w.mask, return_lse=True)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, mask=w.mask)
    torch.cuda.synchronize()
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    var = _variant(w, extras)
    for b, h in ((0, 0), (1, 15)):
        rq, rk, rv, _, _ = oracle.backward_head(q[b, h], k[b, h], v[b, h], do[b, h], f32_scale(w.D), var, b, h, w.Hq)
        check_out(dq[b, h], rq, "bf16", f"dQ[{b},{h}]")
        check_out(dk[b, h], rk, "bf16", f"dK[{b},{h}]")
        check_out(dv[b, h], rv, "bf16", f"dV[{b},{h}]")
