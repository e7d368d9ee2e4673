"""Checks that pin the fp64 oracle to closed forms and invariants.

Each ``check_*`` raises AssertionError when the oracle disagrees with a
result fixed by mathematics (not by re-typing the oracle's formula).  They
take the oracle module as an argument so the mutation tests can run them
against deliberately broken copies.
"""
from __future__ import annotations

import math

import numpy as np

RNG = np.random.default_rng(12345)


def rnd(*shape, rng=None):
    return (rng or RNG).standard_normal(shape)


def close(a, b, tol=1e-10):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(a - b))
    scale = 1.0 + np.where(both_inf, 0.0, np.abs(b))
    worst = float(np.max(err / scale)) if err.size else 0.0
    assert worst <= tol, f"max rel err {worst:.3e} > {tol:.1e}"


def admissible_range(mask, i, window=None, doc=None):
    """Closed form of the admissible key set of query i as a list (contiguous masks)."""
    from synth import MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT
    if mask == MASK_CAUSAL:
        return list(range(0, i + 1))
    if mask == MASK_SLIDING_WINDOW:
        return list(range(max(0, i - window + 1), i + 1))
    if mask == MASK_DOCUMENT:
        start = i
        while start > 0 and doc[start - 1] == doc[i]:
            start -= 1
        return list(range(start, i + 1))
    raise ValueError(mask)


def check_identical_keys(O, mask, S=40, D=6, window=5, scale=0.3):
    """All keys equal => every admissible score of row i is the same number
    c_i, so O_i is the plain mean of the admissible V rows and
    LSE_i = c_i + ln(n_i)."""
    q = rnd(1, 1, S, D)
    k1 = rnd(D)
    k = np.broadcast_to(k1, (1, 1, S, D)).copy()
    v = rnd(1, 1, S, D)
    doc = np.repeat(np.arange(4), [7, 1, 20, 12]).astype(np.int32)[None]
    var = O.Variant(mask=mask, window=window, doc_ids=doc)
    out, lse = O.forward(q, k, v, scale, var)
    for i in range(S):
        if mask == O.MASK_NONE:
            js = list(range(S))
        else:
            js = admissible_range(mask, i, window, doc[0])
        c = scale * float(np.dot(q[0, 0, i], k1))
        close(out[0, 0, i], v[0, 0, js].mean(axis=0))
        close(lse[0, 0, i], c + math.log(len(js)))


def check_single_token(O):
    q, k, v = rnd(1, 1, 1, 8), rnd(1, 1, 1, 8), rnd(1, 1, 1, 8)
    for mask in (O.MASK_NONE, O.MASK_CAUSAL):
        out, lse = O.forward(q, k, v, 0.7, O.Variant(mask=mask))
        close(out[0, 0, 0], v[0, 0, 0])
        close(lse[0, 0, 0], 0.7 * float(np.dot(q[0, 0, 0], k[0, 0, 0])))


def check_causal_row0(O):
    q, k, v = rnd(2, 3, 17, 8), rnd(2, 3, 17, 8), rnd(2, 3, 17, 8)
    out, lse = O.forward(q, k, v, 0.5, O.Variant(mask=O.MASK_CAUSAL))
    close(out[:, :, 0], v[:, :, 0])
    close(lse[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]))


def check_window_edges(O):
    """W = 1 keeps only the diagonal (O_i = V_i); W >= S equals causal."""
    q, k, v = rnd(1, 2, 23, 8), rnd(1, 2, 23, 8), rnd(1, 2, 23, 8)
    out, lse = O.forward(q, k, v, 0.4, O.Variant(mask=O.MASK_SLIDING_WINDOW, window=1))
    close(out, v)
    close(lse, 0.4 * np.einsum("bhsd,bhsd->bhs", q, k))
    a = O.forward(q, k, v, 0.4, O.Variant(mask=O.MASK_SLIDING_WINDOW, window=23))
    b = O.forward(q, k, v, 0.4, O.Variant(mask=O.MASK_CAUSAL))
    close(a[0], b[0])
    close(a[1], b[1])


def check_document_concat(O):
    """Document masking equals running each document as its own causal
    sequence and concatenating; a length-1 document returns its own V row."""
    lens = [5, 1, 9, 3]
    S = sum(lens)
    doc = np.repeat(np.arange(len(lens)), lens).astype(np.int32)[None]
    q, k, v = rnd(1, 2, S, 8), rnd(1, 2, S, 8), rnd(1, 2, S, 8)
    out, lse = O.forward(q, k, v, 0.35, O.Variant(mask=O.MASK_DOCUMENT, doc_ids=doc))
    s0 = 0
    for L in lens:
        sl = slice(s0, s0 + L)
        o2, l2 = O.forward(q[:, :, sl], k[:, :, sl], v[:, :, sl], 0.35, O.Variant(mask=O.MASK_CAUSAL))
        close(out[:, :, sl], o2)
        close(lse[:, :, sl], l2)
        s0 += L
    close(out[:, :, 5], v[:, :, 5])


def check_alibi_geometric(O):
    """Identical keys + causal + ALiBi: the weight of key j in row i is
    r^(i-j) with r = exp(-slope_h), so O_i = sum_m r^m V_{i-m} / sum_m r^m and
    LSE_i = c_i + ln((1 - r^(i+1)) / (1 - r)).  With default slopes this pins
    the sign of the bias and slope_h = 2^(-8(h+1)/Hq)."""
    Hq, S, D = 4, 12, 5
    q = rnd(1, Hq, S, D)
    k1 = rnd(D)
    k = np.broadcast_to(k1, (1, Hq, S, D)).copy()
    v = rnd(1, Hq, S, D)
    out, lse = O.forward(q, k, v, 0.25, O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_ALIBI))
    for h in range(Hq):
        slope = float(np.float32(2.0 ** (-8.0 * (h + 1) / Hq)))
        r = math.exp(-slope)
        for i in range(S):
            w = np.array([r ** (i - j) for j in range(i + 1)])
            expect = (w[:, None] * v[0, h, :i + 1]).sum(0) / ((1 - r ** (i + 1)) / (1 - r))
            close(out[0, h, i], expect, 1e-9)
            c = 0.25 * float(np.dot(q[0, h, i], k1))
            close(lse[0, h, i], c + math.log((1 - r ** (i + 1)) / (1 - r)), 1e-9)


def check_alibi_zero_slope(O):
    q, k, v = rnd(1, 2, 9, 4), rnd(1, 2, 9, 4), rnd(1, 2, 9, 4)
    a = O.forward(q, k, v, 0.5, O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_ALIBI, slopes=np.zeros(2)))
    b = O.forward(q, k, v, 0.5, O.Variant(mask=O.MASK_CAUSAL))
    close(a[0], b[0])
    close(a[1], b[1])


def check_softcap_closed_form(O):
    """tanh(ln 2) = 3/5 exactly.  One query, keys with scores 0 and c ln 2
    under cap c give capped scores 0 and 0.6c, so p_1 = 1/(1 + e^(-0.6c)),
    LSE = ln(1 + e^(0.6c)); the cap's derivative there is 1 - 9/25."""
    c = 2.0
    q = np.ones((1, 1, 1, 1))
    k = np.array([0.0, c * math.log(2.0)]).reshape(1, 1, 2, 1)
    v = np.array([3.0, -5.0]).reshape(1, 1, 2, 1)
    out, lse = O.forward(q, k, v, 1.0, O.Variant(mod=O.MOD_SOFTCAP, softcap=c))
    p1 = 1.0 / (1.0 + math.exp(-0.6 * c))
    close(out[0, 0, 0, 0], (1 - p1) * 3.0 + p1 * -5.0, 1e-13)
    close(lse[0, 0, 0], math.log(1.0 + math.exp(0.6 * c)), 1e-13)
    g = O.modify_grad(O.Variant(mod=O.MOD_SOFTCAP, softcap=c), np.array([[c * math.log(2.0)]]),
                      0, 1, np.array([0]), np.array([0]))
    close(g[0, 0], 16.0 / 25.0, 1e-13)


def check_softcap_limits(O):
    """Identical keys => uniform weights under any monotone cap; a huge cap
    approaches no cap with |c tanh(s/c) - s| <= |s|^3/(3c^2)."""
    S, D = 10, 4
    q = rnd(1, 1, S, D)
    k = np.broadcast_to(rnd(D), (1, 1, S, D)).copy()
    v = rnd(1, 1, S, D)
    out, _ = O.forward(q, k, v, 0.5, O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_SOFTCAP, softcap=0.7))
    for i in range(S):
        close(out[0, 0, i], v[0, 0, :i + 1].mean(0))
    q, k, v = rnd(1, 1, 8, 4), rnd(1, 1, 8, 4), rnd(1, 1, 8, 4)
    a = O.forward(q, k, v, 0.5, O.Variant(mod=O.MOD_SOFTCAP, softcap=1e4))
    b = O.forward(q, k, v, 0.5)
    close(a[0], b[0], 1e-6)


def check_local_boost_two_level(O):
    """Identical keys with common score c: keys with |i-j| < R weigh
    e^(F c), the rest e^c.  R = 3 on 8 tokens makes |i-j| = 3 decide the
    strict inequality."""
    S, D, R, F = 8, 3, 3, 1.1
    q = rnd(1, 1, S, D)
    k1 = rnd(D)
    k = np.broadcast_to(k1, (1, 1, S, D)).copy()
    v = rnd(1, 1, S, D)
    var = O.Variant(mod=O.MOD_LOCAL_BOOST, boost_radius=R, boost_factor=F)
    out, lse = O.forward(q, k, v, 0.8, var)
    for i in range(S):
        c = 0.8 * float(np.dot(q[0, 0, i], k1))
        near = [j for j in range(S) if abs(i - j) <= R - 1]
        far = [j for j in range(S) if abs(i - j) >= R]
        wn, wf = math.exp(F * c), math.exp(c)
        num = wn * v[0, 0, near].sum(0) + wf * v[0, 0, far].sum(0)
        den = wn * len(near) + wf * len(far)
        close(out[0, 0, i], num / den)
        close(lse[0, 0, i], math.log(den))
    for var2 in (O.Variant(mod=O.MOD_LOCAL_BOOST, boost_radius=R, boost_factor=1.0),
                 O.Variant(mod=O.MOD_LOCAL_BOOST, boost_radius=0, boost_factor=F)):
        a, b = O.forward(q, k, v, 0.8, var2), O.forward(q, k, v, 0.8)
        close(a[0], b[0])


def check_invariants(O):
    """Joint permutation of keys and values, a shift of every key (adds a
    per-row constant: O fixed, LSE moves by scale q_i.u), linearity in V and
    rows of P summing to one."""
    q, k, v = rnd(1, 2, 11, 6), rnd(1, 2, 13, 6), rnd(1, 2, 13, 6)
    perm = RNG.permutation(13)
    a = O.forward(q, k, v, 0.45)
    b = O.forward(q, k[:, :, perm], v[:, :, perm], 0.45)
    close(a[0], b[0])
    close(a[1], b[1])
    u = rnd(6)
    for var in (O.Variant(), O.Variant(mask=O.MASK_CAUSAL), O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_ALIBI)):
        qq, kk, vv = q[:, :, :11], k[:, :, :11], v[:, :, :11]
        a = O.forward(qq, kk, vv, 0.45, var)
        b = O.forward(qq, kk + u, vv, 0.45, var)
        close(b[0], a[0])
        close(b[1], a[1] + 0.45 * np.einsum("bhsd,d->bhs", qq, u))
    v2 = rnd(1, 2, 13, 6)
    a = O.forward(q, k, 2.0 * v - 3.0 * v2, 0.45)[0]
    b = 2.0 * O.forward(q, k, v, 0.45)[0] - 3.0 * O.forward(q, k, v2, 0.45)[0]
    close(a, b)
    for mask in (O.MASK_NONE, O.MASK_CAUSAL, O.MASK_SLIDING_WINDOW):
        P = O.probabilities(q[0, 0], k[0, 0, :11], 0.45, O.Variant(mask=mask, window=3))
        close(P.sum(axis=1), np.ones(11), 1e-12)


def check_gqa_equals_repeat(O):
    """GQA equals MHA with each K/V head repeated for its group, forward and
    backward (dK, dV are the group sums)."""
    B, Hq, Hkv, S, D = 1, 6, 2, 9, 4
    q, k, v, do = rnd(B, Hq, S, D), rnd(B, Hkv, S, D), rnd(B, Hkv, S, D), rnd(B, Hq, S, D)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    var = O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_ALIBI)
    a, b = O.forward(q, k, v, 0.5, var), O.forward(q, kr, vr, 0.5, var)
    close(a[0], b[0])
    close(a[1], b[1])
    g1 = O.backward(q, k, v, do, 0.5, var)
    g2 = O.backward(q, kr, vr, do, 0.5, var)
    close(g1[0], g2[0])
    close(g1[1], g2[1].reshape(B, Hkv, G, S, D).sum(2))
    close(g1[2], g2[2].reshape(B, Hkv, G, S, D).sum(2))


VARIANTS_FD = [
    dict(mask=0), dict(mask=1), dict(mask=2, window=3), dict(mask=3),
    dict(mask=1, mod=1), dict(mask=0, mod=2, softcap=1.5), dict(mask=1, mod=3, boost_radius=2, boost_factor=1.1),
    dict(mask=3, mod=2, softcap=2.0),
    dict(mask=0, mod=4, rel_bias=np.random.default_rng(8).standard_normal((2, 13)), rel_origin=6),
]


def check_backward_finite_differences(O, variants=None, h=1e-6, tol=1e-6):
    """Central differences of sum(O * dO) in fp64 on tiny shapes, for every
    element of Q, K and V."""
    B, Hq, Hkv, S, D = 1, 2, 1, 7, 3
    doc = np.repeat(np.arange(3), [2, 1, 4]).astype(np.int32)[None]
    for spec in variants or VARIANTS_FD:
        var = O.Variant(doc_ids=doc, **spec)
        rng = np.random.default_rng(7)
        q, k, v, do = (rnd(B, Hq, S, D, rng=rng), rnd(B, Hkv, S, D, rng=rng),
                       rnd(B, Hkv, S, D, rng=rng), rnd(B, Hq, S, D, rng=rng))
        dq, dk, dv = O.backward(q, k, v, do, 0.6, var)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                old = x[idx]
                x[idx] = old + h
                lp = O.loss(q, k, v, do, 0.6, var)
                x[idx] = old - h
                lm = O.loss(q, k, v, do, 0.6, var)
                x[idx] = old
                num[idx] = (lp - lm) / (2 * h)
            err = np.max(np.abs(num - g)) / (1.0 + np.max(np.abs(g)))
            assert err <= tol, f"{spec}: finite-difference mismatch {err:.2e}"


def check_backward_closed_forms(O):
    """dO = 0 gives zero gradients; with scale 0 and a causal mask P is
    uniform over j <= i, so dQ = dK = 0 and dV_j = sum_{i >= j} dO_i/(i+1)."""
    S, D = 9, 4
    q, k, v, do = rnd(1, 1, S, D), rnd(1, 1, S, D), rnd(1, 1, S, D), rnd(1, 1, S, D)
    g = O.backward(q, k, v, np.zeros_like(do), 0.5, O.Variant(mask=O.MASK_CAUSAL, mod=O.MOD_SOFTCAP, softcap=3.0))
    for x in g:
        close(x, np.zeros_like(x))
    dq, dk, dv = O.backward(q, k, v, do, 0.0, O.Variant(mask=O.MASK_CAUSAL))
    close(dq, np.zeros_like(dq))
    close(dk, np.zeros_like(dk))
    expect = np.stack([sum(do[0, 0, i] / (i + 1) for i in range(j, S)) for j in range(S)])
    close(dv[0, 0], expect)


def check_tile_states(O):
    """Block classification against closed forms: causal with S = n blocks has
    n partial diagonal tiles and n(n-1)/2 full ones; a tile that runs past
    the sequence end is partial even if every in-range pair is admissible; a window of one block width touches two tiles per row; document
    tiles aligned to blocks are full inside a document and empty across."""
    st, kvl, ql = O.tile_states(O.Variant(mask=O.MASK_CAUSAL), 1, 512, 512, 128, 128)
    n = 4
    assert (st[0] == O.TILE_PARTIAL).sum() == n
    assert (st[0] == O.TILE_FULL).sum() == n * (n - 1) // 2
    assert all(list(kvl[0][i]) == list(range(i + 1)) for i in range(n))
    assert all(list(ql[0][j]) == list(range(j, n)) for j in range(n))
    st, _, _ = O.tile_states(O.Variant(mask=O.MASK_CAUSAL), 1, 200, 200, 128, 128)
    assert st[0].tolist() == [[O.TILE_PARTIAL, O.TILE_EMPTY], [O.TILE_PARTIAL, O.TILE_PARTIAL]]
    st, _, _ = O.tile_states(O.Variant(mask=O.MASK_SLIDING_WINDOW, window=128), 1, 512, 512, 128, 128)
    for i in range(4):
        for j in range(4):
            want = O.TILE_PARTIAL if j in (i, i - 1) else O.TILE_EMPTY
            assert st[0, i, j] == want, (i, j, st[0])
    st, _, _ = O.tile_states(O.Variant(mask=O.MASK_NONE), 1, 300, 256, 128, 128)
    assert st[0].tolist() == [[2, 2], [2, 2], [1, 1]]
    doc = np.repeat(np.arange(3), [128, 256, 128]).astype(np.int32)[None]
    st, _, _ = O.tile_states(O.Variant(mask=O.MASK_DOCUMENT, doc_ids=doc), 1, 512, 512, 128, 128)
    want = [[1, 0, 0, 0], [0, 1, 0, 0], [0, 2, 1, 0], [0, 0, 0, 1]]
    assert st[0].tolist() == want, st[0]


def check_pair_counts(O):
    """Admissible pairs: causal S(S+1)/2; window W(W+1)/2 + (S-W)W for S >= W;
    document sum over lengths of L(L+1)/2."""
    S, W = 300, 37
    assert O.count_pairs(O.Variant(mask=O.MASK_CAUSAL), 2, S, S) == 2 * S * (S + 1) // 2
    assert O.count_pairs(O.Variant(mask=O.MASK_SLIDING_WINDOW, window=W), 1, S, S) == W * (W + 1) // 2 + (S - W) * W
    lens = [100, 7, 150, 43]
    doc = np.repeat(np.arange(4), lens).astype(np.int32)[None]
    assert O.count_pairs(O.Variant(mask=O.MASK_DOCUMENT, doc_ids=doc), 1, S, S) == sum(L * (L + 1) // 2 for L in lens)


def _rel_table(rng, Hq, Sq, Skv):
    return rng.standard_normal((Hq, Sq + Skv - 1))


def check_rel_bias_toeplitz(O):
    """Q = 0 makes every scaled score 0, so the weight of key j in row i is
    exp(T_h[i - j + Skv - 1]): a Toeplitz matrix, built here with
    scipy.linalg.toeplitz from its first column (j = 0) and first row
    (i = 0).  O = W V / rowsum(W), LSE = log rowsum(W); causal keeps the
    lower triangle.  Pins the index direction and origin of the table."""
    from scipy.linalg import toeplitz
    rng = np.random.default_rng(21)
    Hq, Sq, Skv, D = 2, 6, 9, 3
    T = _rel_table(rng, Hq, Sq, Skv)
    q = np.zeros((1, Hq, Sq, D))
    k, v = rnd(1, 1, Skv, D, rng=rng), rnd(1, 1, Skv, D, rng=rng)
    o = Skv - 1
    for mask in (O.MASK_NONE, O.MASK_CAUSAL):
        out, lse = O.forward(q, k, v, 0.7, O.Variant(mask=mask, mod=O.MOD_REL_BIAS, rel_bias=T, rel_origin=o))
        for h in range(Hq):
            W = np.exp(toeplitz(T[h, o:o + Sq], T[h, o - np.arange(Skv)]))
            if mask == O.MASK_CAUSAL:
                W = np.tril(W)
            close(out[0, h], (W @ v[0, 0]) / W.sum(1)[:, None], 1e-12)
            close(lse[0, h], np.log(W.sum(1)), 1e-12)


def check_rel_bias_is_alibi(O):
    """A table linear in the relative position, T_h[r] = slope_h (Skv - 1 - r)
    = slope_h (j - i), gives the ALiBi modifier exactly, forward and
    backward."""
    rng = np.random.default_rng(22)
    B, Hq, Hkv, Sq, Skv, D = 1, 4, 2, 7, 9, 3
    slopes = O.default_alibi_slopes(Hq)
    o = Skv - 1
    T = slopes[:, None] * (o - np.arange(Sq + Skv - 1))[None, :]
    q, k, v, do = rnd(B, Hq, Sq, D, rng=rng), rnd(B, Hkv, Skv, D, rng=rng), rnd(B, Hkv, Skv, D, rng=rng), rnd(B, Hq, Sq, D, rng=rng)
    for mask in (O.MASK_NONE, O.MASK_CAUSAL):
        a = O.Variant(mask=mask, mod=O.MOD_ALIBI)
        r = O.Variant(mask=mask, mod=O.MOD_REL_BIAS, rel_bias=T, rel_origin=o)
        for x, y in zip(O.forward(q, k, v, 0.4, a), O.forward(q, k, v, 0.4, r)):
            close(y, x, 1e-12)
        for x, y in zip(O.backward(q, k, v, do, 0.4, a), O.backward(q, k, v, do, 0.4, r)):
            close(y, x, 1e-12)


def check_rel_bias_shift(O):
    """A constant table c_h shifts every admissible score of head h: O and
    dQ, dK, dV are those without a modifier, LSE moves by c_h, and the table
    gradient sums to zero over each head (every row of dS' sums to zero)."""
    rng = np.random.default_rng(23)
    B, Hq, S, D = 2, 2, 8, 4
    c = np.array([0.75, -2.5])
    T = np.repeat(c[:, None], 2 * S - 1, axis=1)
    q, k, v, do = rnd(B, Hq, S, D, rng=rng), rnd(B, Hq, S, D, rng=rng), rnd(B, Hq, S, D, rng=rng), rnd(B, Hq, S, D, rng=rng)
    for mask in (O.MASK_NONE, O.MASK_CAUSAL, O.MASK_SLIDING_WINDOW):
        n = O.Variant(mask=mask, window=3)
        r = O.Variant(mask=mask, window=3, mod=O.MOD_REL_BIAS, rel_bias=T, rel_origin=S - 1)
        (o1, l1), (o2, l2) = O.forward(q, k, v, 0.5, n), O.forward(q, k, v, 0.5, r)
        close(o2, o1, 1e-12)
        close(l2, l1 + c[None, :, None], 1e-12)
        for x, y in zip(O.backward(q, k, v, do, 0.5, n), O.backward(q, k, v, do, 0.5, r)):
            close(y, x, 1e-12)
        g = O.rel_bias_grad(q, k, v, do, 0.5, r)
        assert g.shape == (Hq, 2 * S - 1)
        close(g.sum(1), np.zeros(Hq), 1e-12)
        assert np.abs(g).max() > 1e-3


def check_rel_bias_grad_fd(O, h=1e-6, tol=1e-6):
    """Central differences of sum(O * dO) with respect to every table entry,
    under each mask, with GQA, two batch rows and Sq != Skv."""
    rng = np.random.default_rng(24)
    B, Hq, Hkv, D = 2, 4, 2, 3
    doc = np.array([[0, 0, 1, 1, 1, 2, 2], [0, 1, 1, 1, 1, 1, 2]], dtype=np.int32)
    for mask, Sq, Skv in ((O.MASK_NONE, 5, 7), (O.MASK_CAUSAL, 7, 7), (O.MASK_SLIDING_WINDOW, 7, 7),
                          (O.MASK_DOCUMENT, 7, 7)):
        T = _rel_table(rng, Hq, Sq, Skv)
        var = O.Variant(mask=mask, window=3, doc_ids=doc, mod=O.MOD_REL_BIAS, rel_bias=T, rel_origin=Skv - 1)
        q, k, v, do = rnd(B, Hq, Sq, D, rng=rng), rnd(B, Hkv, Skv, D, rng=rng), rnd(B, Hkv, Skv, D, rng=rng), rnd(B, Hq, Sq, D, rng=rng)
        g = O.rel_bias_grad(q, k, v, do, 0.6, var)
        num = np.zeros_like(T)
        for idx in np.ndindex(T.shape):
            old = T[idx]
            T[idx] = old + h
            lp = O.loss(q, k, v, do, 0.6, var)
            T[idx] = old - h
            lm = O.loss(q, k, v, do, 0.6, var)
            T[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g)) / (1.0 + np.max(np.abs(g)))
        assert err <= tol, f"mask {mask}: table gradient mismatch {err:.2e}"


ALL_CHECKS = [
    check_identical_keys, check_single_token, check_causal_row0, check_window_edges,
    check_document_concat, check_alibi_geometric, check_alibi_zero_slope,
    check_softcap_closed_form, check_softcap_limits, check_local_boost_two_level,
    check_invariants, check_gqa_equals_repeat, check_backward_closed_forms,
    check_tile_states, check_pair_counts,
    check_rel_bias_toeplitz, check_rel_bias_is_alibi, check_rel_bias_shift, check_rel_bias_grad_fd,
]
