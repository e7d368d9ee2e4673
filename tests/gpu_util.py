"""Helpers for the GPU parity tests: device transfer, oracle comparison bars."""
from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

# Tolerances.  bf16 outputs: mean |err| <= 2e-3 and max |err| <= 2e-2 against
# the fp64 oracle, where the max is taken over the error in excess of half a
# bf16 ulp of the exact value: a bf16 output cannot come closer than that
# (at |x| >= 8 the half-ulp is 2^-5 > 2e-2), so only the arithmetic error
# beyond the final rounding is held to 2e-2.  LSE (fp32): relative,
# |err| <= 1e-4 * max(|LSE|, 1/8).  The floor only matters within 1/8 of
# zero, where it is 1.25e-5 absolute: an fp32 LSE = ln2 (m + log2 l) near
# zero cancels m against log2 l and keeps ~|m| 2^-23 of absolute rounding
# error, which no relative bar can hold.  fp32 outputs: the products are exact and the sums run in
# fp32 over at most a few thousand terms, so 1e-4 / 1e-5 leaves two orders
# of margin over the rounding error.
BARS = {
    "bf16": (2e-2, 2e-3),
    "f32": (1e-4, 1e-5),
}
LSE_REL = 1e-4
LSE_FLOOR = 0.125


def dev(t):
    return None if t is None else t.to("cuda").contiguous()


def f32_scale(D: int) -> float:
    return float(ctypes.c_float(1.0 / math.sqrt(D)).value)


def err_stats(got, ref):
    g = got.detach().to("cpu", torch.float64).numpy() if hasattr(got, "detach") else np.asarray(got, np.float64)
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite values in GPU output"
    e = np.abs(g - r)
    return float(e.max(initial=0.0)), float(e.mean()) if e.size else 0.0


def bf16_half_ulp(x):
    """Half the spacing of bf16 numbers at |x| (8 significant bits)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a >= 2.0 ** -126, 2.0 ** (e - 8), 2.0 ** -134)


def check_out(got, ref, dtype: str, what: str = "O", max_excess=None, rounding_mean=False):
    """``rounding_mean``: hold the mean, like the max, to the error beyond
    half a bf16 ulp.  Only for outputs whose magnitude alone puts the mean
    rounding error over the mean bar (e.g. dV of a single key, the sum of
    every dO row: |dV| ~ 11 at 130 rows, where the mean rounding error of
    any bf16 value is ~1e-2)."""
    mx, mean = err_stats(got, ref)
    bmax, bmean = BARS[dtype]
    if max_excess is not None:
        bmax = max_excess
    excess = mx
    if dtype == "bf16":
        g = got.detach().to("cpu", torch.float64).numpy()
        r = np.asarray(ref, dtype=np.float64)
        beyond = np.maximum(np.abs(g - r) - bf16_half_ulp(r), 0.0)
        excess = float(np.max(beyond, initial=0.0))
        if rounding_mean:
            mean = float(beyond.mean()) if beyond.size else 0.0
    assert excess <= bmax and mean <= bmean, (
        f"{what}: max {mx:.3e} (beyond bf16 rounding {excess:.3e}, bar {bmax}), mean {mean:.3e} (bar {bmean})")
    return mx, mean


def check_lse(got, ref, what: str = "LSE", floor: float = LSE_FLOOR):
    """|err| <= 1e-4 max(|LSE|, floor), -inf only where the reference is -inf."""
    g = got.detach().to("cpu", torch.float64).numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape
    both_ninf = np.isneginf(g) & np.isneginf(r)
    assert np.all(np.isfinite(g) | both_ninf), f"{what}: unexpected non-finite values"
    err = np.where(both_ninf, 0.0, np.abs(np.where(both_ninf, 0.0, g) - np.where(both_ninf, 0.0, r)))
    bound = LSE_REL * np.maximum(np.abs(np.where(both_ninf, 0.0, r)), floor)
    worst = float(np.max(err / bound, initial=0.0))
    assert worst <= 1.0, f"{what}: worst |err| / bound = {worst:.3f}"
    return worst
