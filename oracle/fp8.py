"""fp64 CPU oracle for the FP8 forward path.  TEST INFRASTRUCTURE ONLY.

Nothing on the product path may import, call or run this module; it shares
no code with the HIP library.

What the pages say ("FlashAttention-3 (KO)" page, technical innovation 3,
low precision with reduced quantization error): FP8 doubles the speed of
FP16 but loses accuracy to quantization; incoherent processing multiplies
the query and key feature vectors by a random orthogonal matrix (for example
a Hadamard matrix) before quantizing, which spreads outliers over all
coordinates, and because the matrix is orthogonal Q K^T is unchanged; the
page reports about 2.6x lower FP8 attention error than plain FP8.  The page
also lists FP8 as an 8-bit floating-point format.

Readings where the pages are silent (listed in the design notes):
  * The FP8 format is OCP E4M3 (sign, 4 exponent bits with bias 7, 3
    mantissa bits, no infinities, NaN = S.1111.111, largest finite 448,
    subnormals m/8 * 2^-6), rounding to nearest, ties to even, saturating
    at +-448.
  * Non-finite inputs: quantization is elementwise, so a NaN stays NaN (its
    code 0x7F with the sign bit) and +-Inf saturates at +-448 like any value
    out of range; a block's scale comes from its finite values.
  * The random orthogonal matrix is M = diag(s) H_D / sqrt(D): H_D the
    Sylvester Hadamard matrix, s a seeded vector of random signs; rows are
    transformed as x M.  V is not transformed (it is not part of Q K^T).
  * Quantization uses one power-of-two scale per block of 128 rows of one
    (batch, head): the smallest 2^e with max|x| <= 448 * 2^e, stored as the
    byte e + 127 (the E8M0 code); x ~= code value * 2^e.
  * The FP8 forward computes scores from the dequantized Q and K exactly
    (products of FP8 values are exact and accumulate in float32), and
    quantizes the probabilities P of each 64-key step to E4M3 relative to the
    running row max before the P V product; the row sum l takes the
    unrounded probabilities.  That step is an approximation, so
    ``fp8_forward`` follows the online algorithm's steps (the "FlashAttention
    설명" page, §4-§5: running max, rescale by 2^(m_old - m_new), running sum)
    with the rounding of P inserted where the kernel rounds, rather than a
    closed form.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import Variant, allowed, kv_head

E4M3_MAX = 448.0
QBLOCK = 128   # rows per quantization block
FP8_STEP = 64  # keys per step of the FP8 forward


def e4m3_values() -> np.ndarray:
    """Value of every E4M3 code 0..255 (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s, e, m = c >> 7, (c >> 3) & 15, c & 7
        if e == 15 and m == 7:
            v = math.nan
        elif e == 0:
            v = m / 8.0 * 2.0 ** -6
        else:
            v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
        out[c] = -v if s else v
    return out


_VALUES = e4m3_values()
_POS = _VALUES[:127]  # codes 0x00..0x7e: 0 .. 448, strictly increasing


def e4m3_decode(codes) -> np.ndarray:
    return _VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to the even code; saturate at
    +-448 (infinities included); NaN gives the NaN code 0x7F (sign bit of
    the input kept)."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    a = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    hi = np.searchsorted(_POS, a, side="left")          # first value >= a
    hi = np.minimum(hi, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    exact = _POS[hi] == a
    d_lo, d_hi = a - _POS[lo], _POS[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(take_hi, hi, lo)).astype(np.uint8)
    code = np.where(nan, 0x7F, code).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def sylvester(D: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order D (a power of two), entries +-1."""
    h = np.ones((1, 1))
    while h.shape[0] < D:
        h = np.block([[h, h], [h, -h]])
    assert h.shape[0] == D, "D must be a power of two"
    return h


def incoherence_matrix(signs) -> np.ndarray:
    """M = diag(signs) H / sqrt(D), orthogonal."""
    s = np.asarray(signs, dtype=np.float64)
    return (s[:, None] * sylvester(len(s))) / math.sqrt(len(s))


def block_scale_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2^e (0 for amax == 0), clamped
    to the E8M0 range [-127, 127]."""
    if amax == 0.0:
        return 0
    e = math.frexp(amax)[1] - 9  # 2^(e+8) <= amax < 2^(e+9) ... first guess
    while amax > E4M3_MAX * 2.0 ** e:
        e += 1
    while e > -127 and amax <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return max(-127, min(127, e))


def block_quantize(x, signs=None, block: int = QBLOCK):
    """x: [R][S][D].  Returns (codes uint8 [R][S][D], scale bytes uint8
    [R][ceil(S / block)]) with x M ~= decode(codes) * 2^(byte - 127) per block
    (M the incoherence matrix when ``signs`` is given, else the identity)."""
    x = np.asarray(x, dtype=np.float64)
    R, S, D = x.shape
    y = x @ incoherence_matrix(signs) if signs is not None else x
    nb = -(-S // block)
    codes = np.empty((R, S, D), dtype=np.uint8)
    scales = np.empty((R, nb), dtype=np.uint8)
    for r in range(R):
        for b in range(nb):
            blk = y[r, b * block:(b + 1) * block]
            fin = np.abs(blk[np.isfinite(blk)])  # the scale comes from the finite values
            e = block_scale_exponent(float(fin.max()) if fin.size else 0.0)
            scales[r, b] = e + 127
            codes[r, b * block:(b + 1) * block] = e4m3_encode(blk * 2.0 ** -e)
    return codes, scales


def dequantize(codes, scales, block: int = QBLOCK) -> np.ndarray:
    """decode(codes) * 2^(scale - 127), per block of rows."""
    v = e4m3_decode(codes)
    f = np.power(2.0, np.asarray(scales, dtype=np.float64) - 127.0)
    return v * np.repeat(f, block, axis=1)[:, :v.shape[1], None]


def fp8_forward(q8, k8, v8, qs, ks, vs, scale: float, var: Variant | None = None, Hq=None, Hkv=None,
                rows=None, step: int = FP8_STEP):
    """The FP8 forward: q8 [B*Hq][Sq][D], k8/v8 [B*Hkv][Skv][D] codes with
    their block scale bytes.  Returns (O [B*Hq][n_rows][D], LSE [B*Hq][n_rows])
    in float64 for the rows ``rows`` (default all)."""
    var = var or Variant()
    q = dequantize(q8, qs)
    k = dequantize(k8, ks)
    v = dequantize(v8, vs)
    BHq, Sq, D = q.shape
    Skv = k.shape[1]
    Hq = Hq or BHq
    Hkv = Hkv or k.shape[0] * Hq // BHq
    B = BHq // Hq
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    log2e = 1.0 / math.log(2.0)
    O = np.zeros((BHq, len(rows), D))
    L = np.full((BHq, len(rows)), -np.inf)
    for bh in range(BHq):
        b, h = divmod(bh, Hq)
        kh = b * Hkv + kv_head(h, Hq, Hkv)
        x = (q[bh, rows] @ k[kh].T) * scale * log2e          # scores in log2 units
        ok = allowed(var, b, rows, np.arange(Skv))
        x = np.where(ok, x, -np.inf)
        m = np.full(len(rows), -np.inf)
        l = np.zeros(len(rows))
        acc = np.zeros((len(rows), D))
        for j0 in range(0, Skv, step):
            xs = x[:, j0:j0 + step]
            m_new = np.maximum(m, xs.max(axis=1))
            live = m_new > -np.inf
            m_use = np.where(live, m_new, 0.0)
            alpha = np.where(np.isfinite(m), np.exp2(m - m_use), 0.0)
            p = np.exp2(xs - m_use[:, None])                 # 0 where masked
            pq = e4m3_decode(e4m3_encode(p))
            acc = acc * alpha[:, None] + pq @ v[kh, j0:j0 + step]
            l = l * alpha + p.sum(axis=1)
            m = m_new
        nz = l > 0
        O[bh] = np.where(nz[:, None], acc / np.where(nz, l, 1.0)[:, None], 0.0)
        L[bh] = np.where(nz, (m + np.log2(np.where(nz, l, 1.0))) / log2e, -np.inf)
    return O, L
