"""FP8 path on the GPU against the FP8 oracle.

The quantizer is compared with the oracle's quantizer on the same bf16
inputs.  The FP8 forward is fed inputs the oracle quantized (codes and scale
bytes uploaded as they are) and compared with the oracle's emulation of the
FP8 forward, and with the end-to-end claim of the page ("FlashAttention-3
(KO)" page, technical innovation 3): incoherent processing lowers the FP8
attention error.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from oracle import fp8 as ofp8
from tests.gpu_util import bf16_half_ulp, check_lse, f32_scale

pytestmark = pytest.mark.gpu


def _f64(t):
    return t.to(torch.float64).cpu().numpy()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("signed", [False, True])
def test_quantize_matches_oracle(D, signed):
    """Scale bytes equal; codes equal except where the exact transformed value
    sits on an E4M3 rounding midpoint within float32 rounding (the kernel
    transforms in float32): there the two codes are neighbours bracketing it."""
    B, H, S = 2, 3, 300
    g = synth.randn((B, H, S, 1), 71, "f32")
    x = (synth.randn((B, H, S, D), 70, "f32") * torch.exp(g)).to(torch.bfloat16)
    s = synth.signs(D, 72) if signed else None
    x8, sc = fa.quantize_fp8(x.cuda(), None if s is None else s.cuda())
    torch.cuda.synchronize()
    xr = _f64(x).reshape(B * H, S, D)
    codes, scales = ofp8.block_quantize(xr, None if s is None else s.numpy())
    assert np.array_equal(sc.cpu().numpy().reshape(B * H, -1), scales)
    got = x8.cpu().numpy().reshape(B * H, S, D)
    diff = np.argwhere(got != codes)
    assert len(diff) <= max(3, got.size // 10000), len(diff)
    y = xr @ ofp8.incoherence_matrix(s.numpy()) if signed else xr
    vals = ofp8.e4m3_values()
    for r, i, d in diff:
        e = int(scales[r, i // 128]) - 127
        yv = y[r, i, d] * 2.0 ** -e
        a, b = sorted((vals[got[r, i, d]], vals[codes[r, i, d]]))
        assert a <= yv <= b and abs(yv - (a + b) / 2) <= 1e-5 * abs(yv) + 1e-30, (r, i, d, yv, a, b)


def _oracle_quantized(B, Hq, Hkv, S, D, seed, signs):
    q, k, v = synth.qkv(B, Hq, Hkv, S, S, D, seed)
    s = signs.numpy()
    q8, qs = ofp8.block_quantize(_f64(q).reshape(B * Hq, S, D), s)
    k8, ks = ofp8.block_quantize(_f64(k).reshape(B * Hkv, S, D), s)
    v8, vs = ofp8.block_quantize(_f64(v).reshape(B * Hkv, S, D))
    return (q8, qs, k8, ks, v8, vs)


def _gpu_forward(arrs, B, Hq, Hkv, S, D, mask, window):
    q8, qs, k8, ks, v8, vs = (torch.from_numpy(np.ascontiguousarray(a)).cuda() for a in arrs)
    q8, k8, v8 = q8.view(B, Hq, S, D), k8.view(B, Hkv, S, D), v8.view(B, Hkv, S, D)
    o, lse = fa.forward_fp8(q8, k8, v8, qs, ks, vs, scale=f32_scale(D), mask=mask, window=window, return_lse=True)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def _check_fp8_out(o, O, v_absmax):
    """Beyond the bf16 rounding of the output: a rounding flip of one
    probability code (fp32 scores against the oracle's fp64) moves a row by at
    most one E4M3 ulp of that probability, <= 2^-3 * max|v| (p <= 1, l >= 1);
    such flips are rare, so the mean stays near zero."""
    ref = np.asarray(O, dtype=np.float64)
    got = o.to(torch.float64).numpy()
    excess = np.maximum(np.abs(got - ref) - bf16_half_ulp(ref), 0.0)
    assert excess.max() <= 2.0 ** -3 * v_absmax, excess.max()
    assert excess.mean() <= 2e-4, excess.mean()


@pytest.mark.parametrize("mask,window", [(0, 0), (1, 0), (2, 100)])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_forward_matches_oracle(mask, window, D):
    B, Hq, Hkv, S = 2, 4, 2, 333
    arrs = _oracle_quantized(B, Hq, Hkv, S, D, 80 + D, synth.signs(D, 81))
    o, lse = _gpu_forward(arrs, B, Hq, Hkv, S, D, mask, window)
    var = oracle.Variant(mask=mask, window=window)
    O, L = ofp8.fp8_forward(*arrs[0::2], *arrs[1::2], f32_scale(D), var, Hq=Hq, Hkv=Hkv)
    v_absmax = np.abs(ofp8.dequantize(arrs[4], arrs[5])).max()
    _check_fp8_out(o.view(B * Hq, S, D), O, v_absmax)
    check_lse(lse.view(B * Hq, S), L)


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (700, 64)])
@pytest.mark.parametrize("mask,window", [(0, 0), (1, 0), (2, 90)])
def test_fp8_sq_ne_skv(Sq, Skv, mask, window):
    """Unequal query and key lengths (absolute indices; with the window and
    Sq > Skv + window - 1 the last rows have no key: O = 0, LSE = -inf)."""
    B, Hq, Hkv, D = 1, 4, 2, 128
    s = synth.signs(D, 83).numpy()
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, 84)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, 85)
    q8, qs = ofp8.block_quantize(_f64(q).reshape(B * Hq, Sq, D), s)
    k8, ks = ofp8.block_quantize(_f64(k).reshape(B * Hkv, Skv, D), s)
    v8, vs = ofp8.block_quantize(_f64(v).reshape(B * Hkv, Skv, D))

    def gpu(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    o, lse = fa.forward_fp8(gpu(q8).view(B, Hq, Sq, D), gpu(k8).view(B, Hkv, Skv, D), gpu(v8).view(B, Hkv, Skv, D),
                            gpu(qs), gpu(ks), gpu(vs), scale=f32_scale(D), mask=mask, window=window,
                            return_lse=True)
    torch.cuda.synchronize()
    O, L = ofp8.fp8_forward(q8, k8, v8, qs, ks, vs, f32_scale(D), oracle.Variant(mask=mask, window=window),
                            Hq=Hq, Hkv=Hkv)
    _check_fp8_out(o.cpu().view(B * Hq, Sq, D), O, np.abs(ofp8.dequantize(v8, vs)).max())
    check_lse(lse.cpu().view(B * Hq, Sq), L)


def test_fp8_workload_sampled_rows():
    """The FP8 benchmark workload at full size (B2 H16 S8192 D128 causal) on
    256 sampled rows of every head."""
    w = synth.WORKLOADS["causal_fwd_fp8"]
    arrs = _oracle_quantized(w.B, w.Hq, w.Hkv, w.S, w.D, w.seed, synth.signs(w.D, synth.FP8_SIGN_SEED))
    o, lse = _gpu_forward(arrs, w.B, w.Hq, w.Hkv, w.S, w.D, w.mask, 0)
    rows = synth.sample_rows(w.S, 256, w.seed + 7)
    O, L = ofp8.fp8_forward(*arrs[0::2], *arrs[1::2], f32_scale(w.D), oracle.Variant(mask=w.mask), rows=rows)
    v_absmax = np.abs(ofp8.dequantize(arrs[4], arrs[5])).max()
    _check_fp8_out(o.view(w.B * w.Hq, w.S, w.D)[:, rows], O, v_absmax)
    check_lse(lse.view(w.B * w.Hq, w.S)[:, rows], L)


def test_fp8_empty_query_is_noop():
    z = torch.empty((1, 2, 0, 64), dtype=torch.uint8, device="cuda")
    kv = torch.zeros((1, 2, 10, 64), dtype=torch.uint8, device="cuda")
    sc = torch.full((1, 2, 1), 127, dtype=torch.uint8, device="cuda")
    out = fa.forward_fp8(z, kv, kv, sc, sc, sc)
    assert out.shape == (1, 2, 0, 64)


def test_incoherent_processing_lowers_error_end_to_end():
    """GPU quantizer + GPU FP8 forward, with and without the incoherence
    transform, against exact attention on the original inputs (outlier
    features in Q and K, as in the CPU pin): the transform lowers the RMS
    error by at least 1.3x."""
    H, S, D = 2, 512, 128
    rng = np.random.default_rng(0)
    q, k, v = (rng.standard_normal((H, S, D)) for _ in range(3))
    for t in (q, k):
        m = rng.random(t.shape) < 0.001
        t[m] = rng.standard_normal(m.sum()) * 10.0
    qb, kb, vb = (torch.from_numpy(t[None]).to(torch.bfloat16) for t in (q, k, v))
    ref, _ = oracle.forward(_f64(qb), _f64(kb), _f64(vb), f32_scale(D), oracle.Variant(mask=1))
    s = synth.signs(D, 90).cuda()
    rmse = {}
    for name, sg in (("plain", None), ("incoherent", s)):
        q8, qs = fa.quantize_fp8(qb.cuda(), sg)
        k8, ks = fa.quantize_fp8(kb.cuda(), sg)
        v8, vs = fa.quantize_fp8(vb.cuda())
        o = fa.forward_fp8(q8, k8, v8, qs, ks, vs, scale=f32_scale(D), mask=1)
        torch.cuda.synchronize()
        rmse[name] = math.sqrt(np.mean((_f64(o) - ref) ** 2))
    assert rmse["plain"] / rmse["incoherent"] >= 1.3, rmse


@pytest.mark.parametrize("seed", range(700, 712))
def test_fp8_random_case(seed):
    """Seeded random shape, grouping, mask and head dimension, with and
    without incoherent processing."""
    r = np.random.default_rng(seed)
    Hkv = int(r.choice([1, 2, 4]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    B, D = int(r.integers(1, 3)), int(r.choice([64, 128]))
    Sq, Skv = int(r.integers(1, 1200)), int(r.integers(1, 1200))
    mask = int(r.integers(0, 3))
    window = int(r.integers(1, 1300)) if mask == 2 else 0
    s = synth.signs(D, seed).numpy() if r.random() < 0.5 else None
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, seed)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, seed + 1)
    q8, qs = ofp8.block_quantize(_f64(q).reshape(B * Hq, Sq, D), s)
    k8, ks = ofp8.block_quantize(_f64(k).reshape(B * Hkv, Skv, D), s)
    v8, vs = ofp8.block_quantize(_f64(v).reshape(B * Hkv, Skv, D))

    def gpu(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()

    o, lse = fa.forward_fp8(gpu(q8).view(B, Hq, Sq, D), gpu(k8).view(B, Hkv, Skv, D), gpu(v8).view(B, Hkv, Skv, D),
                            gpu(qs), gpu(ks), gpu(vs), scale=f32_scale(D), mask=mask, window=window,
                            return_lse=True)
    torch.cuda.synchronize()
    O, L = ofp8.fp8_forward(q8, k8, v8, qs, ks, vs, f32_scale(D), oracle.Variant(mask=mask, window=window),
                            Hq=Hq, Hkv=Hkv)
    _check_fp8_out(o.cpu().view(B * Hq, Sq, D), O, np.abs(ofp8.dequantize(v8, vs)).max())
    check_lse(lse.cpu().view(B * Hq, Sq), L)
