"""FLOP convention and exact pair counts (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
import synth
from tiled_attention_fa_amd import flops

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "flashinfer_sm120_table.json")


def test_flop_convention_reproduces_page_table():
    """4 D per admissible pair over the query heads reproduces every printed
    TFLOP/s from its printed time, to the 3-digit rounding of the times."""
    table = json.load(open(GOLDEN))
    for B, H, S, D, causal, ms, tflops in table["rows"]:
        n = flops.pairs(flops.MASK_CAUSAL if causal else flops.MASK_NONE, B, H, S, S)
        implied = flops.fwd_flops(n, D) / (ms * 1e-3) / 1e12
        assert abs(implied / tflops - 1.0) < 0.005, (B, H, S, causal, implied, tflops)


def test_halving_convention_would_also_fit():
    """The exact causal count differs from the halved square by a factor (1 + 1/S)."""
    for S in (4096, 8192, 32768):
        assert flops.pairs_per_row_batch(flops.MASK_CAUSAL, S, S) / (S * S / 2) == pytest.approx(1 + 1 / S)


@pytest.mark.parametrize("spec,Sq,Skv", [
    (dict(mask=0), 37, 53), (dict(mask=1), 100, 100), (dict(mask=1), 120, 40), (dict(mask=1), 40, 120),
    (dict(mask=2, window=17), 150, 150), (dict(mask=2, window=500), 150, 150), (dict(mask=2, window=9), 80, 30),
])
def test_pairs_match_brute_force(spec, Sq, Skv):
    want = oracle.count_pairs(oracle.Variant(**spec), 1, Sq, Skv)
    assert flops.pairs_per_row_batch(spec["mask"], Sq, Skv, spec.get("window", 0)) == want


def test_document_pairs_match_brute_force():
    lens = synth.doc_lengths(3000, 1, 400, 5)
    doc = synth.doc_ids_from_lengths(lens)[None]
    want = oracle.count_pairs(oracle.Variant(mask=3, doc_ids=doc), 1, 3000, 3000)
    assert flops.pairs_per_row_batch(3, 3000, 3000, doc_lengths=lens) == want


def test_workload_pair_counts():
    """Exact admissible pairs of the benchmark shapes."""
    w = synth.WORKLOADS
    assert flops.pairs(1, 4, 16, 4096, 4096) == 537_001_984
    assert flops.pairs(1, 2, 32, 8192, 8192) == 2_147_745_792
    assert flops.pairs(2, 2, 32, 8192, 8192, window=1024) == 503_349_248
    assert flops.pairs(1, 2, 16, 8192, 8192) == 1_073_872_896
    d = w["doc_packed"]
    lens = synth.doc_lengths(d.S, 256, 4096, d.seed)
    assert lens.sum() == d.S and lens[:-1].min() >= 256 and lens.max() <= 4096
    n = flops.pairs(3, 1, 16, d.S, d.S, doc_lengths=lens)
    assert n == 16 * int((lens * (lens + 1) // 2).sum())
