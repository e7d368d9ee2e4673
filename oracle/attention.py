"""Plain fp64 CPU oracle for exact attention with masks and score modifiers.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What it computes is the plain definition the pages give, not the tiled
algorithm: the FlashAttention explainer ("FlashAttention 설명", §1 "the real
cost of attention") defines attention as softmax(QK^T/sqrt(d))V over the full
N x N score matrix, and §4 of the same page states that the tiled online
computation gives exactly this result.  So every function here materialises
full score rows in float64, applies the score modifier and the mask, and runs
a two-pass softmax (row max, then normalised exponentials).  Matrix products
use numpy's float64 matmul as a library primitive.

Readings where the pages are silent (each one is listed in the design notes):
  * The modifier acts on the already scaled score, with absolute query and
    key indices, as the FlexAttention score_mod signature (score, b, h, q_idx,
    kv_idx) on the FlexAttention/FA4 page ("섹션별 상세") implies.
  * ALiBi adds slope_h * (j - i) with slope_h = 2^(-8(h+1)/Hq) (query head h),
    rounded to float32 because that is the value the kernel receives.
  * Sliding window keeps keys j with j <= i and i - j < W.
  * Document masking keeps keys with the same document id and j <= i.
  * A row with no admissible key has output 0 and log-sum-exp -inf.
  * GQA maps query head h to key/value head h // (Hq // Hkv).
  * LSE is in natural-log units.
  * The learnable bias (the FlexAttention/FA4 page lists gradients of
    learnable bias tensors among FlexAttention's limits) is a per-query-head
    table of the relative position i - j: the modifier adds
    rel_bias[h][i - j + rel_origin] to the scaled score, with rel_origin =
    Skv - 1 so the table [Hq][Sq + Skv - 1] covers every pair.  ALiBi is the
    case of a linear table.  Its gradient is the sum of dS' (the gradient of
    the modified score) over every (batch, i, j) that reads the entry.
The backward pass is not on the pages; it is the chain rule of the same
definition (see ``backward_head``).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT = 0, 1, 2, 3
MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_LOCAL_BOOST, MOD_REL_BIAS = 0, 1, 2, 3, 4
TILE_EMPTY, TILE_PARTIAL, TILE_FULL = 0, 1, 2


@dataclasses.dataclass
class Variant:
    """Mask and score-modifier choice with their parameters."""
    mask: int = MASK_NONE
    window: int = 0
    doc_ids: np.ndarray | None = None      # int [B, S] document id per token
    mod: int = MOD_NONE
    slopes: np.ndarray | None = None       # [Hq]; None -> default ALiBi slopes
    softcap: float = 0.0
    boost_radius: int = 0
    boost_factor: float = 1.0
    rel_bias: np.ndarray | None = None     # [Hq][Sq + Skv - 1] (MOD_REL_BIAS)
    rel_origin: int = 0                    # index of relative position 0: Skv - 1


def default_alibi_slopes(Hq: int) -> np.ndarray:
    """slope_h = 2^(-8(h+1)/Hq), rounded to float32 and widened back."""
    h = np.arange(Hq, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / Hq).astype(np.float32).astype(np.float64)


def allowed(var: Variant, b: int, i: np.ndarray, j: np.ndarray) -> np.ndarray:
    """Boolean [len(i), len(j)]: may query i attend to key j (absolute indices)."""
    I = np.asarray(i, dtype=np.int64)[:, None]
    J = np.asarray(j, dtype=np.int64)[None, :]
    if var.mask == MASK_NONE:
        return np.ones((I.shape[0], J.shape[1]), dtype=bool)
    if var.mask == MASK_CAUSAL:
        return J <= I
    if var.mask == MASK_SLIDING_WINDOW:
        return (J <= I) & (I - J < var.window)
    if var.mask == MASK_DOCUMENT:
        doc = np.asarray(var.doc_ids[b], dtype=np.int64)
        return (doc[I] == doc[J]) & (J <= I)
    raise ValueError(f"unknown mask kind {var.mask}")


def modify(var: Variant, s: np.ndarray, h: int, Hq: int, i: np.ndarray, j: np.ndarray) -> np.ndarray:
    """Score modifier applied to the scaled score s[i, j]."""
    if var.mod == MOD_NONE:
        return s
    I = np.asarray(i, dtype=np.float64)[:, None]
    J = np.asarray(j, dtype=np.float64)[None, :]
    if var.mod == MOD_ALIBI:
        slopes = default_alibi_slopes(Hq) if var.slopes is None else np.asarray(var.slopes, np.float64)
        return s + slopes[h] * (J - I)
    if var.mod == MOD_SOFTCAP:
        c = float(var.softcap)
        return c * np.tanh(s / c)
    if var.mod == MOD_LOCAL_BOOST:
        near = np.abs(I - J) < var.boost_radius
        return np.where(near, s * float(var.boost_factor), s)
    if var.mod == MOD_REL_BIAS:
        return s + np.asarray(var.rel_bias, dtype=np.float64)[h][rel_index(var, i, j)]
    raise ValueError(f"unknown score modifier {var.mod}")


def rel_index(var: Variant, i, j) -> np.ndarray:
    """Table index i - j + rel_origin of every pair, [len(i), len(j)]."""
    return np.asarray(i, dtype=np.int64)[:, None] - np.asarray(j, dtype=np.int64)[None, :] + int(var.rel_origin)


def modify_grad(var: Variant, s: np.ndarray, h: int, Hq: int, i: np.ndarray, j: np.ndarray) -> np.ndarray:
    """d modify / d s, elementwise."""
    if var.mod in (MOD_NONE, MOD_ALIBI, MOD_REL_BIAS):
        return np.ones_like(s)
    if var.mod == MOD_SOFTCAP:
        t = np.tanh(s / float(var.softcap))
        return 1.0 - t * t
    if var.mod == MOD_LOCAL_BOOST:
        I = np.asarray(i, dtype=np.float64)[:, None]
        J = np.asarray(j, dtype=np.float64)[None, :]
        near = np.abs(I - J) < var.boost_radius
        return np.where(near, float(var.boost_factor), 1.0) * np.ones_like(s)
    raise ValueError(f"unknown score modifier {var.mod}")


def kv_head(h: int, Hq: int, Hkv: int) -> int:
    """Key/value head serving query head h: contiguous groups of Hq // Hkv."""
    return h // (Hq // Hkv)


def _f64(x) -> np.ndarray:
    """Exact widening of a bf16/f32 torch tensor or array to float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch  # local: only for the dtype conversion of torch inputs
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(sm: np.ndarray, ok: np.ndarray):
    """Two-pass softmax of each row over its admissible entries.

    Returns (P, M, Z): probabilities, row max and row normaliser.  Rows with
    no admissible entry get P = 0, M = -inf, Z = 0.
    """
    x = np.where(ok, sm, -np.inf)
    M = np.max(x, axis=1) if x.shape[1] else np.full(x.shape[0], -np.inf)
    empty = ~np.isfinite(M)
    Msafe = np.where(empty, 0.0, M)
    E = np.where(ok, np.exp(x - Msafe[:, None]), 0.0)
    Z = E.sum(axis=1)
    P = E / np.where(empty, 1.0, Z)[:, None]
    return P, M, Z


def score_rows(q_rows, k_head, scale, var, b, h, Hq, rows, Skv):
    """Scaled scores, modified scores and admissibility for the given rows."""
    cols = np.arange(Skv)
    s = scale * (q_rows @ k_head.T)
    sm = modify(var, s, h, Hq, rows, cols)
    ok = allowed(var, b, rows, cols)
    return s, sm, ok


def forward(q, k, v, scale: float, var: Variant | None = None, rows=None, block: int = 1024):
    """Attention output and LSE.

    q [B,Hq,Sq,D], k and v [B,Hkv,Skv,D] (any dtype; widened exactly).
    ``rows``: optional sorted query indices; only those rows are computed
    (each row is an exact, independent check).  Returns (O [B,Hq,R,D],
    LSE [B,Hq,R]) in float64.
    """
    var = var or Variant()
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, D = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    O = np.zeros((B, Hq, len(rows), v.shape[3]))
    LSE = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            hk = kv_head(h, Hq, Hkv)
            for r0 in range(0, len(rows), block):
                rr = rows[r0:r0 + block]
                _, sm, ok = score_rows(q[b, h, rr], k[b, hk], scale, var, b, h, Hq, rr, Skv)
                P, M, Z = _softmax_rows(sm, ok)
                O[b, h, r0:r0 + len(rr)] = P @ v[b, hk]
                with np.errstate(divide="ignore"):
                    LSE[b, h, r0:r0 + len(rr)] = np.where(Z > 0, M + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    return O, LSE


def probabilities(q_head, k_head, scale, var, b=0, h=0, Hq=1):
    """Full softmax matrix P [Sq, Skv] of one head (small sizes; for checks)."""
    q_head, k_head = _f64(q_head), _f64(k_head)
    rows = np.arange(q_head.shape[0])
    _, sm, ok = score_rows(q_head, k_head, scale, var, b, h, Hq, rows, k_head.shape[0])
    return _softmax_rows(sm, ok)[0]


def backward_head(q_h, k_h, v_h, do_h, scale, var, b, h, Hq, check_delta: bool = True, with_dsp: bool = False):
    """Gradients of sum(O * dO) for one query head, by the chain rule.

    With s = scale q k^T, s' = mod(s), P = softmax over admissible keys and
    O = P V:  dV = P^T dO,  dP = dO V^T,  D_i = sum_j P_ij dP_ij,
    dS'_ij = P_ij (dP_ij - D_i),  dS = dS' * mod'(s),  dQ = scale dS K,
    dK = scale dS^T Q.  D_i is also formed as dO_i . O_i and the two must
    agree.  Returns (dq, dk, dv, O, LSE) for this head; dk and dv are this
    query head's share of its key/value head's gradient.  ``with_dsp`` appends
    dS' [Sq, Skv], the gradient of the modified scores (zero where masked).
    """
    q_h, k_h, v_h, do_h = _f64(q_h), _f64(k_h), _f64(v_h), _f64(do_h)
    Sq, Skv = q_h.shape[0], k_h.shape[0]
    rows, cols = np.arange(Sq), np.arange(Skv)
    s, sm, ok = score_rows(q_h, k_h, scale, var, b, h, Hq, rows, Skv)
    P, M, Z = _softmax_rows(sm, ok)
    O = P @ v_h
    dV = P.T @ do_h
    dP = do_h @ v_h.T
    Dsum = np.sum(P * dP, axis=1)
    if check_delta:
        Ddot = np.sum(do_h * O, axis=1)
        tol = 1e-9 * (1.0 + np.abs(Ddot).max(initial=0.0))
        assert np.allclose(Dsum, Ddot, rtol=1e-9, atol=tol), "D_i two ways disagree"
    dSp = P * (dP - Dsum[:, None])
    dS = dSp * modify_grad(var, s, h, Hq, rows, cols)
    dQ = scale * (dS @ k_h)
    dK = scale * (dS.T @ q_h)
    with np.errstate(divide="ignore"):
        LSE = np.where(Z > 0, M + np.log(np.where(Z > 0, Z, 1.0)), -np.inf)
    if with_dsp:
        return dQ, dK, dV, O, LSE, dSp
    return dQ, dK, dV, O, LSE


def backward(q, k, v, do, scale: float, var: Variant | None = None, heads=None):
    """dQ [B,Hq,Sq,D], dK and dV [B,Hkv,Skv,D] (summed over each GQA group).

    ``heads``: optional list of (b, hq) query heads to include; dq rows of the
    other heads stay zero and dk/dv hold only the listed heads' shares.
    """
    var = var or Variant()
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, D = q.shape
    Hkv = k.shape[1]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in todo:
        hk = kv_head(h, Hq, Hkv)
        gq, gk, gv, _, _ = backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, var, b, h, Hq)
        dq[b, h] = gq
        dk[b, hk] += gk
        dv[b, hk] += gv
    return dq, dk, dv


def rel_bias_grad(q, k, v, do, scale: float, var: Variant, heads=None) -> np.ndarray:
    """Gradient of sum(O * dO) with respect to the MOD_REL_BIAS table
    [Hq][Sq + Skv - 1].  The table entry r enters the modified score of
    every pair (b, i, j) with i - j + rel_origin = r, with derivative 1, so
    its gradient is the sum of dS'_bij over those pairs (np.add.at does the
    scatter-sum).  ``heads``: optional list of (b, hq) to include."""
    q, k, v, do = _f64(q), _f64(k), _f64(v), _f64(do)
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = np.zeros((Hq, Sq + Skv - 1))
    rows, cols = np.arange(Sq), np.arange(Skv)
    todo = [(b, h) for b in range(B) for h in range(Hq)] if heads is None else list(heads)
    for b, h in todo:
        hk = kv_head(h, Hq, Hkv)
        dSp = backward_head(q[b, h], k[b, hk], v[b, hk], do[b, h], scale, var, b, h, Hq, with_dsp=True)[5]
        np.add.at(G[h], rel_index(var, rows, cols), dSp)
    return G


def loss(q, k, v, do, scale, var=None):
    """sum(O * dO): the scalar whose gradient ``backward`` returns."""
    O, _ = forward(q, k, v, scale, var)
    return float(np.sum(O * _f64(do)))


def count_pairs(var: Variant, B: int, Sq: int, Skv: int, block: int = 2048) -> int:
    """Number of admissible (query, key) pairs summed over the batch, by brute force."""
    total = 0
    cols = np.arange(Skv)
    for b in range(B if var.mask == MASK_DOCUMENT else 1):
        for r0 in range(0, Sq, block):
            total += int(allowed(var, b, np.arange(r0, min(Sq, r0 + block)), cols).sum())
    if var.mask != MASK_DOCUMENT:
        total *= B
    return total


def tile_states(var: Variant, B: int, Sq: int, Skv: int, bq: int, bkv: int):
    """Brute-force block mask.

    Each bq x bkv tile is EMPTY if no in-range element is admissible, FULL if
    every element is in range and admissible, PARTIAL otherwise.  Returns
    (state [nb, nq, nkv] uint8, kv lists, q lists) where nb = B for document
    masks and 1 otherwise, kv lists[b][qt] are the ascending non-empty kv
    tiles of each query tile and q lists[b][kt] the ascending non-empty query
    tiles of each kv tile.
    """
    nq, nkv = -(-Sq // bq), -(-Skv // bkv)
    nb = B if var.mask == MASK_DOCUMENT else 1
    st = np.zeros((nb, nq, nkv), dtype=np.uint8)
    for b in range(nb):
        for qt in range(nq):
            rows = np.arange(qt * bq, min(Sq, (qt + 1) * bq))
            a = allowed(var, b, rows, np.arange(Skv))
            for kt in range(nkv):
                blk = a[:, kt * bkv:min(Skv, (kt + 1) * bkv)]
                inrange = blk.shape == (bq, bkv)
                if not blk.any():
                    st[b, qt, kt] = TILE_EMPTY
                elif blk.all() and inrange:
                    st[b, qt, kt] = TILE_FULL
                else:
                    st[b, qt, kt] = TILE_PARTIAL
    kv_lists = [[np.nonzero(st[b, qt])[0].astype(np.int32) for qt in range(nq)] for b in range(nb)]
    q_lists = [[np.nonzero(st[b, :, kt])[0].astype(np.int32) for kt in range(nkv)] for b in range(nb)]
    return st, kv_lists, q_lists


def logsumexp_row_fsum(values) -> float:
    """log(sum(exp(x))) of a short list by exact summation (math.fsum)."""
    vals = [float(x) for x in values]
    if not vals:
        return -math.inf
    m = max(vals)
    return m + math.log(math.fsum(math.exp(x - m) for x in vals))
