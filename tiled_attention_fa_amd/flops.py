"""Work counts for attention: admissible (query, key) pairs and FLOPs.

Convention ("FlashInfer SM120 NVFP4 어텐션 최적화" page, §1 benchmark script
and the performance table): forward FLOPs = 4 * D per admissible pair,
counted over the query/output heads, i.e. 4 B Hq S^2 D without a mask and
half that when causal.  This module counts admissible pairs exactly
(S(S+1)/2 for causal), which differs from the halved square by 1/S.  The
backward pass is counted as 10 * D per pair (five D-long contractions:
the recomputed Q K^T, dO V^T, P^T dO, dS K and dS^T Q) - a reading, since
the pages give no backward count.
"""
from __future__ import annotations

import numpy as np

MASK_NONE, MASK_CAUSAL, MASK_SLIDING_WINDOW, MASK_DOCUMENT = 0, 1, 2, 3


def pairs_per_row_batch(mask: int, Sq: int, Skv: int, window: int = 0, doc_lengths=None) -> int:
    """Admissible pairs of one (batch row, head)."""
    if mask == MASK_NONE:
        return Sq * Skv
    i = np.arange(Sq, dtype=np.int64)
    hi = np.minimum(i, Skv - 1)  # last admissible key (causal part)
    if mask == MASK_CAUSAL:
        return int(np.maximum(hi + 1, 0).sum())
    if mask == MASK_SLIDING_WINDOW:
        lo = np.maximum(i - window + 1, 0)
        return int(np.maximum(hi - lo + 1, 0).sum())
    if mask == MASK_DOCUMENT:
        L = np.asarray(doc_lengths, dtype=np.int64)
        return int((L * (L + 1) // 2).sum())
    raise ValueError(mask)


def pairs(mask: int, B: int, Hq: int, Sq: int, Skv: int, window: int = 0, doc_lengths=None) -> int:
    """Admissible pairs over the batch and the query heads."""
    return B * Hq * pairs_per_row_batch(mask, Sq, Skv, window, doc_lengths)


def fwd_flops(npairs: int, D: int) -> float:
    return 4.0 * D * npairs


def bwd_flops(npairs: int, D: int) -> float:
    return 10.0 * D * npairs
