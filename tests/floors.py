"""The bf16 floor of a backward pass: the error that remains when the fp64
chain rule takes exactly the roundings the method's data path imposes and
nothing else.  The forward's output O reaches the backward as bf16 (it is an
input of fa_bwd), so delta = rowsum(dO * O) uses the rounded O; dS is a bf16
operand of the dQ and dK contractions and P one of the dV contraction.  A
bf16-operand backward cannot be more accurate than this on the same case.
Errors are measured beyond half a bf16 ulp of the exact value, as the parity
checks measure them (CPU only, through the oracle)."""
import numpy as np
import torch

import oracle
from oracle import attention as oa
from tests.gpu_util import bf16_half_ulp


def _bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()


def _beyond(rounded, exact):
    return float(np.max(np.maximum(np.abs(rounded - exact) - bf16_half_ulp(exact), 0.0), initial=0.0))


def backward_floors(q, k, v, do, scale, var):
    """(dQ, dK, dV) floors of one case: q [B,Hq,Sq,D], k/v [B,Hkv,Skv,D]."""
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    rows, cols = np.arange(Sq), np.arange(Skv)
    dq_e, dq_r = np.zeros((B, Hq, Sq, D)), np.zeros((B, Hq, Sq, D))
    dk_e, dk_r = np.zeros((B, Hkv, Skv, D)), np.zeros((B, Hkv, Skv, D))
    dv_e, dv_r = np.zeros((B, Hkv, Skv, D)), np.zeros((B, Hkv, Skv, D))
    for b in range(B):
        for h in range(Hq):
            hk = h // G
            Q, K, V, dO = (t.double().numpy() for t in (q[b, h], k[b, hk], v[b, hk], do[b, h]))
            s, sm, ok = oa.score_rows(Q, K, scale, var, b, h, Hq, rows, Skv)
            P = oa._softmax_rows(sm, ok)[0]
            grad = oa.modify_grad(var, s, h, Hq, rows, cols)
            dP = dO @ V.T
            O = P @ V
            dS = P * (dP - np.sum(dO * O, axis=1)[:, None]) * grad
            dS_r = _bf16(P * (dP - np.sum(dO * _bf16(O), axis=1)[:, None]) * grad)
            dq_e[b, h], dq_r[b, h] = scale * dS @ K, scale * dS_r @ K
            dk_e[b, hk] += scale * dS.T @ Q
            dk_r[b, hk] += scale * dS_r.T @ Q
            dv_e[b, hk] += P.T @ dO
            dv_r[b, hk] += _bf16(P).T @ dO
    return _beyond(dq_r, dq_e), _beyond(dk_r, dk_e), _beyond(dv_r, dv_e)


def rounding_mean(exact):
    """Mean |bf16(x) - x| over an exact output: what rounding the result to
    bf16 alone adds to the mean error, before any arithmetic error."""
    x = np.asarray(exact, dtype=np.float64)
    return float(np.mean(np.abs(_bf16(x) - x))) if x.size else 0.0
