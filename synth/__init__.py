"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This module holds input generation only: random tensors, document lengths,
sampled row sets and the table of benchmark shapes.  It contains none of the
attention arithmetic, so both the GPU path and the CPU oracle may use it
without sharing any of the method's code.

Recipe (fixed, so every run sees the same bits):
  * Q, K, V, dO are float32 N(0, 1) drawn from a CPU ``torch.Generator``
    seeded with ``seed``, then rounded to bfloat16 with round-to-nearest-even
    (``Tensor.to(torch.bfloat16)``).  The fp32 workload keeps float32.
  * Tensors too large to draw at once (``randn_chunked``) are filled in
    chunks of 2^24 values, each from its own seeded generator.
  * Document lengths are integers drawn uniformly from [lo, hi] inclusive with
    ``numpy.random.default_rng(seed)`` until their sum reaches the packed
    length; the last one is cut so the sum is exact.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT = 0, 1, 2, 3
MOD_NONE, MOD_ALIBI, MOD_SOFTCAP, MOD_LOCAL_BOOST = 0, 1, 2, 3

_DTYPES = {"bf16": torch.bfloat16, "f32": torch.float32}


def randn(shape, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """N(0,1) float32 from a seeded CPU generator, rounded (RNE) to ``dtype``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    return x.to(_DTYPES[dtype]).contiguous()


def randn_chunked(shape, seed: int, dtype: str = "bf16", chunk: int = 1 << 24) -> torch.Tensor:
    """Like ``randn`` for very large tensors: the flattened tensor is filled
    in chunks of ``chunk`` values, chunk c drawn from a CPU generator seeded
    with ``seed * 1000003 + c``, so no float32 copy of the whole tensor is
    ever held.  (Different values from ``randn`` with the same seed.)"""
    out = torch.empty(int(np.prod(shape)), dtype=_DTYPES[dtype])
    g = torch.Generator(device="cpu")
    for c, lo in enumerate(range(0, out.numel(), chunk)):
        n = min(chunk, out.numel() - lo)
        g.manual_seed(int(seed) * 1000003 + c)
        out[lo:lo + n] = torch.randn(n, generator=g, dtype=torch.float32).to(_DTYPES[dtype])
    return out.view(*shape)


def qkv(B, Hq, Hkv, Sq, Skv, D, seed: int, dtype: str = "bf16"):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Skv,D] from three derived seeds."""
    q = randn((B, Hq, Sq, D), seed, dtype)
    k = randn((B, Hkv, Skv, D), seed + 1, dtype)
    v = randn((B, Hkv, Skv, D), seed + 2, dtype)
    return q, k, v


def rel_bias_table(Hq: int, Sq: int, Skv: int, seed: int, std: float = 1.0) -> torch.Tensor:
    """A relative-position bias table [Hq, Sq + Skv - 1]: float32 N(0, std^2)
    from a seeded CPU generator (entry i - j + Skv - 1 belongs to query i and
    key j)."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return (torch.randn(Hq, max(Sq + Skv - 1, 0), generator=g, dtype=torch.float32) * std).contiguous()


def doc_lengths(total: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Packed document lengths: uniform integers in [lo, hi], last one truncated."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return np.asarray(out, dtype=np.int64)


def doc_ids_from_lengths(lengths) -> np.ndarray:
    """int32 document id per token, ascending from 0."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), np.asarray(lengths))


def sample_rows(S: int, n: int, seed: int, extra=()) -> np.ndarray:
    """Sorted unique query rows: the first and last 128, ``extra`` boundary
    rows (each with its neighbours), and seeded uniform rows up to ``n``."""
    rows = set(range(min(128, S)))
    rows.update(range(max(0, S - 128), S))
    for e in extra:
        for d in (-1, 0, 1):
            if 0 <= e + d < S:
                rows.add(int(e + d))
    rng = np.random.default_rng(seed)
    while len(rows) < min(n, S):
        rows.add(int(rng.integers(0, S)))
    return np.asarray(sorted(rows), dtype=np.int64)


@dataclasses.dataclass(frozen=True)
class Workload:
    """One benchmark shape.  ``mask``/``mod`` use the constants above."""
    name: str
    B: int
    Hq: int
    Hkv: int
    S: int
    D: int
    dtype: str
    mask: int = MASK_NONE
    mod: int = MOD_NONE
    window: int = 0
    softcap: float = 0.0
    boost_radius: int = 0
    boost_factor: float = 1.0
    lse: bool = False
    backward: bool = False
    doc_range: tuple = ()
    seed: int = 0


def signs(D: int, seed: int) -> torch.Tensor:
    """Seeded vector of random +-1 (float32 [D]): the diagonal of the random
    orthogonal matrix of the FP8 path's incoherent processing."""
    g = torch.Generator().manual_seed(seed)
    return (torch.randint(0, 2, (D,), generator=g) * 2 - 1).to(torch.float32)


# The five workload families: a tiny fp32 MHA check, a causal prefill, GQA
# with the four score-mod/mask variants, a packed document batch and a causal
# forward+backward.  Seeds are 1000 + family index.
WORKLOADS = {
    "tiny_mha_f32": Workload("tiny_mha_f32", 1, 2, 2, 256, 64, "f32", lse=True, seed=1000),
    "causal_prefill": Workload("causal_prefill", 4, 16, 16, 4096, 128, "bf16",
                               mask=MASK_CAUSAL, lse=True, seed=1001),
    "gqa_alibi": Workload("gqa_alibi", 2, 32, 8, 8192, 128, "bf16", mask=MASK_CAUSAL,
                          mod=MOD_ALIBI, lse=True, seed=1002),
    "gqa_softcap": Workload("gqa_softcap", 2, 32, 8, 8192, 128, "bf16", mask=MASK_CAUSAL,
                            mod=MOD_SOFTCAP, softcap=30.0, lse=True, seed=1002),
    "gqa_window": Workload("gqa_window", 2, 32, 8, 8192, 128, "bf16",
                           mask=MASK_SLIDING_WINDOW, window=1024, lse=True, seed=1002),
    "gqa_boost": Workload("gqa_boost", 2, 32, 8, 8192, 128, "bf16", mod=MOD_LOCAL_BOOST,
                          boost_radius=128, boost_factor=1.1, lse=True, seed=1002),
    "gqa_causal": Workload("gqa_causal", 2, 32, 8, 8192, 128, "bf16", mask=MASK_CAUSAL,
                           lse=True, seed=1002),
    "doc_packed": Workload("doc_packed", 1, 16, 16, 32768, 128, "bf16", mask=MASK_DOCUMENT,
                           lse=True, doc_range=(256, 4096), seed=1003),
    "causal_fwd_bwd": Workload("causal_fwd_bwd", 2, 16, 16, 8192, 128, "bf16",
                               mask=MASK_CAUSAL, lse=True, backward=True, seed=1004),
    # The FP8 forward (E4M3 Q, K, V; Q and K with incoherent processing) at
    # the causal S=8192 shape.
    "causal_fwd_fp8": Workload("causal_fwd_fp8", 2, 16, 16, 8192, 128, "fp8",
                               mask=MASK_CAUSAL, lse=True, seed=1005),
}

FP8_SIGN_SEED = 2005  # seed of the incoherence signs of the FP8 workloads


def workload_inputs(w: Workload, dtype: str | None = None):
    """(q, k, v, extras) CPU tensors for a workload; extras holds dO and doc ids.
    FP8 workloads start from bf16 tensors (quantized by the caller)."""
    dt = dtype or ("bf16" if w.dtype == "fp8" else w.dtype)
    q, k, v = qkv(w.B, w.Hq, w.Hkv, w.S, w.S, w.D, w.seed, dt)
    extras = {}
    if w.backward:
        extras["do"] = randn((w.B, w.Hq, w.S, w.D), w.seed + 100, dt)
    if w.mask == MASK_DOCUMENT:
        lens = doc_lengths(w.S, w.doc_range[0], w.doc_range[1], w.seed)
        extras["doc_lengths"] = lens
        ids = doc_ids_from_lengths(lens)
        extras["doc_ids"] = torch.from_numpy(np.tile(ids, (w.B, 1))).contiguous()
    return q, k, v, extras
