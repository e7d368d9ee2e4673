"""fa_bwd_noalloc (the backward whose workspace is the library's fixed
device scratch, for callers that cannot allocate) against fa_bwd with a
caller workspace: identical bits on two calls in a row, the second smaller
than the first (the scratch keeps the first call's contents), and the size
limit is rejected on the host."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import dev, f32_scale

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, S, D, spec, seed):
    q, k, v = synth.qkv(B, Hq, Hkv, S, S, D, seed)
    do = synth.randn((B, Hq, S, D), seed + 100)
    qd, kd, vd, dod = dev(q), dev(k), dev(v), dev(do)
    o, lse = fa.forward(qd, kd, vd, scale=f32_scale(D), return_lse=True, **spec)
    return qd, kd, vd, o, dod, lse


def _grads_like(q, k):
    return torch.full_like(q, float("nan")), torch.full_like(k, float("nan")), torch.full_like(k, float("nan"))


def _same_bits(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("spec", [dict(mask=1), dict(mask=2, window=300, mod=1), dict(mask=0, mod=2, softcap=30.0)])
def test_noalloc_matches_fa_bwd_twice_shrinking(spec):
    big = _case(2, 8, 4, 1500, 128, spec, 31)
    small = _case(1, 4, 2, 333, 64, spec, 32)
    for qd, kd, vd, o, dod, lse in (big, small):
        ref = fa.backward(qd, kd, vd, o, dod, lse, scale=f32_scale(qd.shape[-1]), **spec)
        got = _grads_like(qd, kd)
        fa.backward(qd, kd, vd, o, dod, lse, scale=f32_scale(qd.shape[-1]), grads=got, noalloc=True, **spec)
        torch.cuda.synchronize()
        for g, r, what in zip(got, ref, ("dQ", "dK", "dV")):
            assert _same_bits(g, r), what


def test_noalloc_rejects_oversize_before_launch():
    """B * Hq * Sq above 2^21 rows needs more workspace than the fixed
    scratch: rejected on the host (no tensor is touched, so fake pointers
    serve)."""
    P = ctypes.c_void_p(0x100000)
    rows = (fa.FA_NOALLOC_SCRATCH_BYTES // 8) + 256
    B, Hq, S = 1, 16, rows // 16
    mp, op = fa.FaMaskParams(0, None, None), fa.FaModParams(None, 1.0, 0, 1.0, None, None, None, 0)
    rc = fa.fa_bwd_noalloc(P, P, P, P, P, P, P, P, P, B, Hq, Hq, S, S, 128, fa.FA_BF16, 0.088, 1,
                           ctypes.byref(mp), 0, ctypes.byref(op), None, None)
    assert rc == fa.FA_ERR_SCRATCH
    assert fa.fa_bwd_workspace_bytes(B, Hq, S, 128) > fa.FA_NOALLOC_SCRATCH_BYTES
    # the largest size that fits is accepted by the size check (bad pointer
    # alignment is reported instead, so nothing launches)
    S2 = (fa.FA_NOALLOC_SCRATCH_BYTES // 8) // 16
    MIS = ctypes.c_void_p(0x100008)
    rc2 = fa.fa_bwd_noalloc(MIS, P, P, P, P, P, P, P, P, B, Hq, Hq, S2, S2, 128, fa.FA_BF16, 0.088, 1,
                            ctypes.byref(mp), 0, ctypes.byref(op), None, None)
    assert rc2 == fa.FA_ERR_ALIGN


def test_noalloc_inside_graph_capture():
    """Captured into a HIP graph (nothing allocates during capture) and
    replayed: every replay equals the eager fa_bwd result."""
    qd, kd, vd, o, dod, lse = _case(1, 4, 4, 700, 128, dict(mask=1), 33)
    ref = fa.backward(qd, kd, vd, o, dod, lse, mask=1)
    got = _grads_like(qd, kd)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fa.backward(qd, kd, vd, o, dod, lse, mask=1, grads=got, noalloc=True, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fa.backward(qd, kd, vd, o, dod, lse, mask=1, grads=got, noalloc=True)
    other = _case(1, 2, 2, 200, 64, dict(mask=0), 34)
    for rep in range(3):
        for t in got:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b, what in zip(got, ref, ("dQ", "dK", "dV")):
            assert _same_bits(a, b), (rep, what)
        # eager work between replays, through the same scratch
        fa.backward(*other, mask=0, noalloc=True)
        torch.cuda.synchronize()
