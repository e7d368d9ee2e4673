"""The stored-dS backward: with a workspace of fa_bwd_ds_workspace_bytes the
dK/dV launch also writes its bf16 dS tiles and the dQ launch computes
dQ = scale dS K from them instead of recomputing the scores and dO V^T
(no mask or the causal mask).  Checked against the fp64 oracle at the same
bars as the recomputing path, for determinism and phase order, and by
reading the stored tiles back out of the workspace and comparing them with
the oracle's dS, which pins their layout."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.floors import backward_floors, rounding_mean
from tests.gpu_util import bf16_half_ulp, check_out, dev, f32_scale

pytestmark = pytest.mark.gpu

MODS = {"none": {}, "alibi": dict(mod=1), "softcap": dict(mod=2, softcap=30.0),
        "boost": dict(mod=3, boost_radius=96, boost_factor=1.1)}


def _run(B, Hq, Hkv, Sq, Skv, D, spec, seed, workspace=None):
    q, _, _ = synth.qkv(B, Hq, Hkv, Sq, Sq, D, seed)
    _, k, v = synth.qkv(B, Hq, Hkv, Skv, Skv, D, seed + 1)
    do = synth.randn((B, Hq, Sq, D), seed + 2)
    scale = f32_scale(D)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(qd, kd, vd, scale=scale, return_lse=True, **spec)
    got = fa.backward(qd, kd, vd, o, dod, lse, scale=scale, store_ds=True, workspace=workspace, **spec)
    torch.cuda.synchronize()
    return (q, k, v, do, scale), got


def _check(inputs, got, spec, what_prefix=""):
    q, k, v, do, scale = inputs
    var = oracle.Variant(**spec)
    ref = oracle.backward(q, k, v, do, scale, var)
    floors = backward_floors(q, k, v, do, scale, var)
    for g, r, what, fl in zip(got, ref, ("dQ", "dK", "dV"), floors):
        check_out(g, r, "bf16", f"{what_prefix}{what} floor {fl:.2e}", max_excess=max(2e-2, 1.5 * fl),
                  rounding_mean=rounding_mean(r) > 1e-3)


@pytest.mark.parametrize("mod", sorted(MODS))
@pytest.mark.parametrize("mask", [0, 1])
@pytest.mark.parametrize("D", [64, 128])
def test_stored_ds_variants(mod, mask, D):
    spec = dict(mask=mask, **MODS[mod])
    inputs, got = _run(1, 4, 2, 333, 333, D, spec, 60 + D + mask)
    _check(inputs, got, spec)


@pytest.mark.parametrize("Sq,Skv", [(200, 333), (333, 200), (64, 700), (700, 64), (1, 300), (300, 1), (1300, 1300)])
@pytest.mark.parametrize("mask", [0, 1])
def test_stored_ds_lengths(Sq, Skv, mask):
    """Unequal and ragged lengths (absolute causal indices), one long case."""
    spec = dict(mask=mask)
    inputs, got = _run(1, 2, 1, Sq, Skv, 128, spec, Sq + 7 * Skv)
    _check(inputs, got, spec, f"{Sq}x{Skv} ")


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 2), (8, 1)])
def test_stored_ds_grouping(Hq, Hkv):
    spec = dict(mask=1, mod=1)
    inputs, got = _run(2, Hq, Hkv, 260, 260, 128, spec, 70 + Hkv)
    _check(inputs, got, spec)


def test_stored_ds_deterministic_and_phases():
    """Two calls give the same bits, and DELTA, DKDV, DQ one at a time on one
    stream equal the single call."""
    B, Hq, Hkv, S, D = 1, 4, 2, 700, 128
    q, k, v = (dev(t) for t in synth.qkv(B, Hq, Hkv, S, S, D, 80))
    do = dev(synth.randn((B, Hq, S, D), 81))
    o, lse = fa.forward(q, k, v, mask=1, return_lse=True)
    a = fa.backward(q, k, v, o, do, lse, mask=1, store_ds=True)
    b = fa.backward(q, k, v, o, do, lse, mask=1, store_ds=True)
    ws = torch.empty(fa.fa_bwd_ds_workspace_bytes(B, Hq, S, S, D, 1), dtype=torch.uint8, device="cuda")
    grads = tuple(torch.empty_like(t) for t in a)
    for ph in (fa.FA_BWD_DELTA, fa.FA_BWD_DKDV, fa.FA_BWD_DQ):
        fa.backward(q, k, v, o, do, lse, mask=1, workspace=ws, grads=grads, phases=ph)
    torch.cuda.synchronize()
    for x, y, z in zip(a, b, grads):
        assert torch.equal(x, y) and torch.equal(x, z)


def _ds_block(mask, kt, qs, n_qs):
    if mask == 1:
        m = min(kt, (n_qs + 3) // 4)
        return m * n_qs - 2 * m * (m - 1) + (qs - 4 * kt)
    return kt * n_qs + qs


@pytest.mark.parametrize("mask", [0, 1])
def test_stored_tiles_equal_oracle_ds(mask):
    """The workspace (filled with NaN first) holds, after the call, bf16 dS
    in blocks of 32 query rows x 128 keys: element (wave w, lane l, r) of
    block (key tile kt, query step qs) is dS[32 qs + 8 (r / 4) + 4 (l / 32) +
    r % 4][128 kt + 32 w + l % 32].  Every stored pair is compared with the
    oracle's dS (beyond half a bf16 ulp, the output bar), masked pairs must
    be zero, and so is the whole 32-key piece of a wave that skips a step."""
    B, Hq, Hkv, Sq, Skv, D = 1, 2, 1, 300, 280, 64
    ws = torch.full((fa.fa_bwd_ds_workspace_bytes(B, Hq, Sq, Skv, D, mask),), 0xFF, dtype=torch.uint8,
                    device="cuda")
    inputs, got = _run(B, Hq, Hkv, Sq, Skv, D, dict(mask=mask), 90, workspace=ws)
    q, k, v, do, scale = inputs
    base = 2 * (-(-(B * Hq * Sq * 4) // 256) * 256)
    tiles = ws[base:].view(torch.bfloat16).to(torch.float64).cpu().numpy()
    n_qs, n_kt = -(-Sq // 32), -(-Skv // 128)
    blocks = _ds_block(mask, n_kt, 4 * n_kt if mask == 1 else 0, n_qs)
    assert tiles.size == B * Hq * blocks * 4096
    tiles = tiles.reshape(B * Hq, blocks, 4, 64, 16)
    var = oracle.Variant(mask=mask)
    w_, l_, r_ = np.meshgrid(np.arange(4), np.arange(64), np.arange(16), indexing="ij")
    rows_in = 8 * (r_ // 4) + 4 * (l_ // 32) + r_ % 4
    keys_in = 32 * w_ + l_ % 32
    for h in range(Hq):
        dsp = oracle.backward_head(q[0, h], k[0, 0], v[0, 0], do[0, h], scale, var, 0, h, Hq, with_dsp=True)[5]
        for kt in range(n_kt):
            for qs in range(4 * kt if mask == 1 else 0, n_qs):
                blk = tiles[h, _ds_block(mask, kt, qs, n_qs)]
                assert np.all(np.isfinite(blk)), (h, kt, qs)
                i, j = 32 * qs + rows_in, 128 * kt + keys_in
                inside = (i < Sq) & (j < Skv)
                exact = np.where(inside, dsp[np.minimum(i, Sq - 1), np.minimum(j, Skv - 1)], 0.0)
                beyond = np.maximum(np.abs(blk - exact) - bf16_half_ulp(exact), 0.0)
                assert beyond.max() <= 2e-2, (h, kt, qs, beyond.max())
