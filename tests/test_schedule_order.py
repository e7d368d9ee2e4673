"""The block-mask schedule order's rule (tests/test_block_mask.py checks the
library's orders against it on the GPU): under a document mask, a
permutation that keeps each document's tiles together, heaviest document
first and longest tile first inside it; where every list starts (ends) at
the same tile it is the plain longest-first order."""
import numpy as np
import pytest

import oracle
import synth
from tests.test_block_mask import expected_order


def _lists(var, S):
    _, kvl, ql = oracle.tile_states(var, 1, S, S, 128, 128)
    n = -(-S // 128)

    def dense(ls):
        cnt = np.array([len(x) for x in ls])
        arr = np.full((len(ls), n), -1)
        for t, x in enumerate(ls):
            arr[t, :len(x)] = x
        return cnt, arr
    return dense(kvl[0]), dense(ql[0])


@pytest.mark.parametrize("spec", [dict(mask=0), dict(mask=1)])
def test_one_group_is_longest_first(spec):
    """Causal and unmasked q lists all start at kv tile 0 (and kv lists end
    at the last q tile): one group, so grouping changes nothing."""
    (kc, ki), (qc, qi) = _lists(oracle.Variant(**spec), 1500)
    for cnt, lists, first in ((kc, ki, True), (qc, qi, False)):
        plain = sorted(range(len(cnt)), key=lambda t: (-cnt[t], t))
        assert expected_order(cnt, lists, first) == plain
        assert expected_order(cnt, lists, first, documents=False) == plain


def test_documents_stay_together():
    ids = synth.doc_ids_from_lengths(synth.doc_lengths(8192, 256, 2048, 7))
    (kc, ki), (qc, qi) = _lists(oracle.Variant(mask=3, doc_ids=ids[None]), 8192)
    order = expected_order(kc, ki, True)
    assert sorted(order) == list(range(len(kc)))
    first = [int(ki[t, 0]) for t in order]
    # Each group (first kv tile) occupies one contiguous run of positions.
    runs = [g for i, g in enumerate(first) if i == 0 or g != first[i - 1]]
    assert len(runs) == len(set(runs))
    # Heaviest group first, and longest first inside each group.
    w = [max(kc[t] for t in order if ki[t, 0] == g) for g in runs]
    assert w == sorted(w, reverse=True)
    for g in runs:
        c = [kc[t] for t in order if ki[t, 0] == g]
        assert c == sorted(c, reverse=True)
