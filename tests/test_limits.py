"""The largest sequences the library accepts, checked with closed forms that
hold at any length (the oracle's dense rows are too slow at millions of keys).

* Forward at the maximum length, 4,194,304 tokens (causal, one head, LSE).
  K is zero except for 2048 seeded random rows R, so a zero key j scores
  exactly 0 and row i reduces to: random keys R_i = R n [0, i] with scores
  s_j = scale q_i . k_j, plus z_i = i + 1 - |R_i| keys of score 0 whose values
  sum to (V_0 + ... + V_i) - sum_{j in R_i} V_j.  With m = max(s_j, 0):
      O_i   = (sum_R e^(s_j - m) V_j + e^(-m) sum_zero V_j) / Z,
      Z     = sum_R e^(s_j - m) + z_i e^(-m),     LSE_i = m + ln Z.
  A key or value read from the wrong row moves a random key's weight onto
  another value and fails the check.
* Forward and backward at 262,144 and 4,194,304 tokens with identical keys.  Every score
  of row i is the same number c_i = scale q_i . k, so under the causal mask
  P_ij = 1/(i+1) for j <= i and:
      O_i   = mean of V_0..V_i,       LSE_i = c_i + ln(i + 1),
      dV_j  = sum_{i>=j} dO_i / (i+1),
      dQ_i  = scale k sum_j dS_ij = 0  (each row of dS sums to zero),
      dK_j  = scale (M_j V_j - c_j),  M_j = sum_{i>=j} q_i dO_i^T / (i+1),
                                      c_j = sum_{i>=j} (dO_i . O_i) q_i / (i+1).
  The sums over i >= j are suffix sums, evaluated at the sampled keys.
"""
import numpy as np
import pytest
import torch

import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import check_lse, check_out, f32_scale

pytestmark = pytest.mark.gpu

MAX_SEQ = 1 << 22  # the library's limit on Sq and Skv


def _prefix_sums_at(x: torch.Tensor, rows: np.ndarray, chunk: int = 1 << 18) -> np.ndarray:
    """fp64 sums x[0] + ... + x[i] for each ascending row i of ``rows``."""
    out = np.zeros((len(rows), x.shape[1]))
    run = np.zeros(x.shape[1])
    r = 0
    for lo in range(0, x.shape[0], chunk):
        c = x[lo:lo + chunk].to(torch.float64).numpy()
        pos = 0
        while r < len(rows) and rows[r] < lo + len(c):
            end = rows[r] - lo + 1
            run = run + c[pos:end].sum(axis=0)
            out[r], pos, r = run, end, r + 1
        run = run + c[pos:].sum(axis=0)
    return out


def test_forward_max_sequence_sparse_keys():
    S, D = MAX_SEQ, 128
    scale = f32_scale(D)
    rng = np.random.default_rng(4242)
    R = np.unique(np.concatenate([[0, 1, S // 2, S - 2, S - 1], rng.integers(0, S, 2043)]))
    q = synth.randn_chunked((1, 1, S, D), 4243)
    v = synth.randn_chunked((1, 1, S, D), 4244)
    kr = synth.randn((len(R), D), 4245)
    k = torch.zeros(1, 1, S, D, dtype=torch.bfloat16)
    k[0, 0, torch.from_numpy(R)] = kr
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), mask=fa.MASK_CAUSAL, return_lse=True)
    torch.cuda.synchronize()

    rows = np.unique(np.concatenate([np.arange(64), np.arange(S - 64, S), R[::64], R[::64] - 1,
                                     rng.integers(0, S, 64)]))
    rows = rows[rows >= 0]
    pv = _prefix_sums_at(v[0, 0], rows)
    KR = kr.to(torch.float64).numpy()
    VR = v[0, 0, torch.from_numpy(R)].to(torch.float64).numpy()
    Qr = q[0, 0, torch.from_numpy(rows)].to(torch.float64).numpy()
    O_ref = np.zeros((len(rows), D))
    L_ref = np.zeros(len(rows))
    for t, i in enumerate(rows):
        n_r = int(np.searchsorted(R, i, side="right"))  # keys of R at or before i
        s = scale * (KR[:n_r] @ Qr[t])
        z = i + 1 - n_r
        m = max(s.max(initial=-np.inf), 0.0 if z > 0 else -np.inf)
        w = np.exp(s - m)
        Z = w.sum() + z * np.exp(-m)
        O_ref[t] = (w @ VR[:n_r] + np.exp(-m) * (pv[t] - VR[:n_r].sum(axis=0))) / Z
        L_ref[t] = m + np.log(Z)
    check_out(o.cpu()[0, 0, torch.from_numpy(rows)], O_ref, "bf16")
    check_lse(lse.cpu()[0, 0, torch.from_numpy(rows)], L_ref)


def _suffix_at(sorted_js, S, seg_sum):
    """Suffix sums F(j) = sum_{i >= j} f(i) at ascending ``sorted_js``;
    ``seg_sum(a, b)`` returns sum_{a <= i < b} f(i)."""
    out, acc, hi = [None] * len(sorted_js), None, S
    for n in range(len(sorted_js) - 1, -1, -1):
        part = seg_sum(sorted_js[n], hi)
        acc = part if acc is None else acc + part
        out[n] = acc
        hi = sorted_js[n]
    return out


@pytest.mark.parametrize("S", [1 << 18, MAX_SEQ])
def test_identical_keys_forward_backward_long(S):
    D = 128
    scale = f32_scale(D)
    q = synth.randn_chunked((1, 1, S, D), 777)
    v = synth.randn_chunked((1, 1, S, D), 778)
    do = synth.randn_chunked((1, 1, S, D), 779)
    k = synth.randn((1, 1, 1, D), 780).expand(1, 1, S, D).contiguous()
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, mask=fa.MASK_CAUSAL, return_lse=True)
    dq, dk, dv = fa.backward(qd, kd, vd, o, dod, lse, mask=fa.MASK_CAUSAL)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu()[0, 0] for t in (o, lse, dq, dk, dv))

    Q, K, V, dO = (t[0, 0].to(torch.float64).numpy() for t in (q, k, v, do))
    n = np.arange(1, S + 1, dtype=np.float64)[:, None]  # i + 1
    O_ref = np.cumsum(V, axis=0) / n
    check_out(o, O_ref, "bf16", "O")
    check_lse(lse, scale * (Q @ K[0]) + np.log(n[:, 0]))
    check_out(dq, np.zeros((S, D)), "bf16", "dQ")

    js = np.unique(np.concatenate([np.arange(128), np.arange(S - 128, S), 97 * 256 * np.arange(1, 40) % S,
                                   np.random.default_rng(9).integers(0, S, 64)]))
    w = 1.0 / n  # 1 / (i + 1)
    Dl = np.einsum("id,id->i", dO, O_ref)[:, None]
    dV_ref = _suffix_at(js, S, lambda a, b: (dO[a:b] * w[a:b]).sum(axis=0))
    M = _suffix_at(js, S, lambda a, b: (Q[a:b] * w[a:b]).T @ dO[a:b])
    cc = _suffix_at(js, S, lambda a, b: (Q[a:b] * (Dl[a:b] * w[a:b])).sum(axis=0))
    dK_ref = np.stack([scale * (M[t] @ V[j] - cc[t]) for t, j in enumerate(js)])
    check_out(dv[js], np.stack(dV_ref), "bf16", "dV")
    check_out(dk[js], dK_ref, "bf16", "dK")
