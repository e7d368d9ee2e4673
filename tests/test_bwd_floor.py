"""Why two backward cases get a wider bar than 2e-2 on dK (and dV).

The kernels feed dS to the dK contraction and P to the dV contraction as
bf16 (the MFMA operand type).  These tests round only that operand to bf16
in the fp64 oracle's chain rule, keep everything else exact, and measure the
error beyond half a bf16 ulp of the exact value (the same measure the parity
tests use).  In the exempted cases |dK| reaches ~10-12 and |dV| ~24 (many
rows put their weight on the same keys) and this rounding alone costs most
of, or more than, the 2e-2 bar, before any fp32 accumulation error: no
bf16-operand backward can meet 2e-2 there.  The inputs are those of the
parity tests (same seeds and shapes).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import bf16_half_ulp, f32_scale


def dv_floor(q, k, v, do, D, spec):
    Hq, Hkv = q.shape[1], k.shape[1]
    G, Sq, Skv = Hq // Hkv, q.shape[2], k.shape[2]
    scale, var = f32_scale(D), oracle.Variant(**spec)
    exact = np.zeros((Hkv, Skv, D))
    rounded = np.zeros((Hkv, Skv, D))
    for h in range(Hq):
        hk = h // G
        P = oracle.probabilities(q[0, h], k[0, hk], scale, var, 0, h, Hq)
        dO = do[0, h].double().numpy()
        exact[hk] += P.T @ dO
        rounded[hk] += torch.from_numpy(P).to(torch.bfloat16).double().numpy().T @ dO
    return float(np.max(np.maximum(np.abs(rounded - exact) - bf16_half_ulp(exact), 0.0)))


def dk_floor(q, k, v, do, D, spec):
    Hq, Hkv = q.shape[1], k.shape[1]
    G, Sq, Skv = Hq // Hkv, q.shape[2], k.shape[2]
    scale, var = f32_scale(D), oracle.Variant(**spec)
    exact = np.zeros((Hkv, Skv, D))
    rounded = np.zeros((Hkv, Skv, D))
    for h in range(Hq):
        hk = h // G
        dsp = oracle.backward_head(q[0, h], k[0, hk], v[0, hk], do[0, h], scale, var, 0, h, Hq, with_dsp=True)[5]
        qh = q[0, h].double().numpy()
        exact[hk] += scale * (dsp.T @ qh)  # ALiBi and no modifier: dS = dS'
        rounded[hk] += scale * (torch.from_numpy(dsp).to(torch.bfloat16).double().numpy().T @ qh)
    return float(np.max(np.maximum(np.abs(rounded - exact) - bf16_half_ulp(exact), 0.0)))


@pytest.mark.parametrize("D", [64, 128])
def test_none_alibi_333(D):
    q, k, v = synth.qkv(1, 4, 2, 333, 333, D, 21)
    do = synth.randn((1, 4, 333, D), 121)
    assert dk_floor(q, k, v, do, D, dict(mask=0, mod=1)) > 1.5e-2


@pytest.mark.parametrize("D", [64, 128])
def test_causal_alibi_700_queries_64_keys(D):
    q, _, _ = synth.qkv(1, 4, 2, 700, 700, D, 40)
    _, k, v = synth.qkv(1, 4, 2, 64, 64, D, 41)
    do = synth.randn((1, 4, 700, D), 42)
    assert dk_floor(q, k, v, do, D, dict(mask=1, mod=1)) > 1.5e-2
    assert dv_floor(q, k, v, do, D, dict(mask=1, mod=1)) > 2e-2
