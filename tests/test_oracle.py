"""The fp64 oracle against closed forms and invariants (CPU only).

The mutation tests plant plausible mistakes in the oracle (on the CPU) and
check that at least one pin fails for each, so a pin is known to bite.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as OA
from tests import oracle_pins as pins

MASKS = [oracle.MASK_NONE, oracle.MASK_CAUSAL, oracle.MASK_SLIDING_WINDOW, oracle.MASK_DOCUMENT]


@pytest.mark.parametrize("mask", MASKS)
def test_identical_keys(mask):
    pins.check_identical_keys(oracle, mask)


def test_identical_keys_zero_scale():
    """scale = 0 makes every score equal, like identical keys."""
    for mask in MASKS:
        pins.check_identical_keys(oracle, mask, scale=0.0)


@pytest.mark.parametrize("check", pins.ALL_CHECKS[1:], ids=lambda f: f.__name__)
def test_pin(check):
    check(oracle)


def test_backward_finite_differences():
    pins.check_backward_finite_differences(oracle)


def test_lse_matches_exact_sum():
    """LSE of sampled rows equals log-sum-exp of the admissible modified
    scores accumulated with math.fsum (an independent summation)."""
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((1, 2, 20, 5)), rng.standard_normal((1, 1, 20, 5)), rng.standard_normal((1, 1, 20, 5))
    var = oracle.Variant(mask=oracle.MASK_CAUSAL, mod=oracle.MOD_ALIBI)
    _, lse = oracle.forward(q, k, v, 0.3, var)
    slopes = oracle.default_alibi_slopes(2)
    for h in range(2):
        for i in (0, 7, 19):
            vals = [0.3 * float(np.dot(q[0, h, i], k[0, 0, j])) + slopes[h] * (j - i) for j in range(i + 1)]
            assert abs(lse[0, h, i] - oracle.logsumexp_row_fsum(vals)) < 1e-12


def test_empty_rows_defined():
    """Skv = 0: every row is empty, O = 0 and LSE = -inf."""
    q = np.ones((1, 1, 3, 4))
    k = np.ones((1, 1, 0, 4))
    out, lse = oracle.forward(q, k, k, 0.5)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- mutations

def _bad_window_le(var, b, i, j):
    I, J = np.asarray(i)[:, None], np.asarray(j)[None, :]
    if var.mask == oracle.MASK_SLIDING_WINDOW:
        return (J <= I) & (I - J <= var.window)
    return _orig_allowed(var, b, i, j)


def _bad_doc_no_causal(var, b, i, j):
    if var.mask == oracle.MASK_DOCUMENT:
        d = np.asarray(var.doc_ids[b])
        return d[np.asarray(i)][:, None] == d[np.asarray(j)][None, :]
    return _orig_allowed(var, b, i, j)


def _bad_alibi_sign(var, s, h, Hq, i, j):
    if var.mod == oracle.MOD_ALIBI:
        sl = oracle.default_alibi_slopes(Hq) if var.slopes is None else np.asarray(var.slopes)
        return s + sl[h] * (np.asarray(i)[:, None] - np.asarray(j)[None, :])
    return _orig_modify(var, s, h, Hq, i, j)


def _bad_alibi_head(var, s, h, Hq, i, j):
    if var.mod == oracle.MOD_ALIBI and var.slopes is None:
        sl = oracle.default_alibi_slopes(Hq)
        return s + sl[Hq - 1 - h] * (np.asarray(j)[None, :] - np.asarray(i)[:, None])
    return _orig_modify(var, s, h, Hq, i, j)


def _bad_boost_le(var, s, h, Hq, i, j):
    if var.mod == oracle.MOD_LOCAL_BOOST:
        near = np.abs(np.asarray(i)[:, None] - np.asarray(j)[None, :]) <= var.boost_radius
        return np.where(near, s * var.boost_factor, s)
    return _orig_modify(var, s, h, Hq, i, j)


def _bad_softcap_grad(var, s, h, Hq, i, j):
    return np.ones_like(s)


def _bad_kv_head(h, Hq, Hkv):
    return h % Hkv


def _bad_rel_direction(var, s, h, Hq, i, j):
    if var.mod == oracle.MOD_REL_BIAS:
        T = np.asarray(var.rel_bias)
        idx = (np.asarray(j)[None, :] - np.asarray(i)[:, None] + var.rel_origin) % T.shape[1]
        return s + T[h][idx]
    return _orig_modify(var, s, h, Hq, i, j)


def _bad_rel_origin(var, s, h, Hq, i, j):
    if var.mod == oracle.MOD_REL_BIAS:
        T = np.asarray(var.rel_bias)
        return s + T[h][(OA.rel_index(var, i, j) + 1) % T.shape[1]]
    return _orig_modify(var, s, h, Hq, i, j)


def _bad_rel_grad_transposed(q, k, v, do, scale, var, heads=None):
    """Scatters dS'_ij to entry j - i + origin instead of i - j + origin."""
    g = _orig_rel_bias_grad(q, k, v, do, scale, var, heads)
    return g[:, ::-1].copy()


def _bad_rel_grad_no_delta(q, k, v, do, scale, var, heads=None):
    """Forms the table gradient from P dP, dropping the - D_i term."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    B, Hq, Sq, _ = q.shape
    Hkv, Skv = k.shape[1], k.shape[2]
    G = np.zeros((Hq, Sq + Skv - 1))
    rows, cols = np.arange(Sq), np.arange(Skv)
    for b in range(B):
        for h in range(Hq):
            hk = OA.kv_head(h, Hq, Hkv)
            _, sm, ok = OA.score_rows(q[b, h], k[b, hk], scale, var, b, h, Hq, rows, Skv)
            P = OA._softmax_rows(sm, ok)[0]
            np.add.at(G[h], OA.rel_index(var, rows, cols), P * (do[b, h] @ v[b, hk].T))
    return G


_orig_allowed = OA.allowed
_orig_modify = OA.modify
_orig_rel_bias_grad = OA.rel_bias_grad

MUTATIONS = {
    "window_le": ("allowed", _bad_window_le),
    "document_not_causal": ("allowed", _bad_doc_no_causal),
    "alibi_sign": ("modify", _bad_alibi_sign),
    "alibi_head_order": ("modify", _bad_alibi_head),
    "boost_le": ("modify", _bad_boost_le),
    "softcap_grad_dropped": ("modify_grad", _bad_softcap_grad),
    "gqa_interleaved_heads": ("kv_head", _bad_kv_head),
    "rel_bias_direction": ("modify", _bad_rel_direction),
    "rel_bias_origin": ("modify", _bad_rel_origin),
    "rel_bias_grad_transposed": ("rel_bias_grad", _bad_rel_grad_transposed),
    "rel_bias_grad_no_delta": ("rel_bias_grad", _bad_rel_grad_no_delta),
}


def _all_pins_pass():
    for mask in MASKS:
        pins.check_identical_keys(OA, mask)
    for check in pins.ALL_CHECKS[1:]:
        check(OA)
    pins.check_backward_finite_differences(OA, variants=[pins.VARIANTS_FD[5], pins.VARIANTS_FD[7]])


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(OA, attr, fn)
    with pytest.raises(AssertionError):
        _all_pins_pass()


def test_pins_catch_transposed_dk(monkeypatch):
    """A backward that forms dK from dS instead of dS^T is caught by finite differences."""
    def bad(q_h, k_h, v_h, do_h, scale, var, b, h, Hq, check_delta=True):
        q_h, k_h, v_h, do_h = (np.asarray(x, dtype=np.float64) for x in (q_h, k_h, v_h, do_h))
        rows, cols = np.arange(q_h.shape[0]), np.arange(k_h.shape[0])
        s, sm, ok = OA.score_rows(q_h, k_h, scale, var, b, h, Hq, rows, k_h.shape[0])
        P, M, Z = OA._softmax_rows(sm, ok)
        dP = do_h @ v_h.T
        dS = P * (dP - np.sum(P * dP, axis=1)[:, None]) * OA.modify_grad(var, s, h, Hq, rows, cols)
        return scale * (dS @ k_h), scale * (dS @ q_h), P.T @ do_h, P @ v_h, M + np.log(Z)

    monkeypatch.setattr(OA, "backward_head", bad)
    with pytest.raises(AssertionError):
        pins.check_backward_finite_differences(OA, variants=[pins.VARIANTS_FD[1]])
