"""Block-mask builder and tile skipping: bit-exact against brute force."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tiled_attention_fa_amd as fa
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

CASES = [
    (dict(mask=0), 1, 300, 300),
    (dict(mask=0), 1, 256, 640),
    (dict(mask=1), 1, 1000, 1000),
    (dict(mask=1), 1, 200, 700),
    (dict(mask=2, window=128), 1, 900, 900),
    (dict(mask=2, window=300), 1, 777, 777),
    (dict(mask=2, window=1), 1, 513, 513),
    (dict(mask=3), 2, 1500, 1500),
    (dict(mask=3), 1, 4096, 4096),
]


def _docs(B, S, seed, lo=1, hi=None):
    hi = hi or max(2, S // 4)
    return torch.from_numpy(np.stack([synth.doc_ids_from_lengths(synth.doc_lengths(S, lo, hi, seed + b))
                                      for b in range(B)])).to(torch.int32)


@pytest.mark.parametrize("case", range(len(CASES)))
def test_builder_matches_brute_force(case):
    spec, B, Sq, Skv = CASES[case]
    doc = _docs(B, Sq, 40 + case) if spec["mask"] == 3 else None
    bm = fa.build_block_mask(spec["mask"], B, Sq, Skv, window=spec.get("window", 0), doc_ids=dev(doc))
    torch.cuda.synchronize()
    var = oracle.Variant(doc_ids=None if doc is None else doc.numpy(), **spec)
    st, kvl, ql = oracle.tile_states(var, B, Sq, Skv, 128, 128)
    assert np.array_equal(bm.tile_state.cpu().numpy(), st)
    kc, ki = bm.kv_count.cpu().numpy(), bm.kv_index.cpu().numpy()
    qc, qi = bm.q_count.cpu().numpy(), bm.q_index.cpu().numpy()
    for b in range(st.shape[0]):
        for t in range(st.shape[1]):
            n = len(kvl[b][t])
            assert kc[b, t] == n and np.array_equal(ki[b, t, :n], kvl[b][t]) and np.all(ki[b, t, n:] == -1)
        for t in range(st.shape[2]):
            n = len(ql[b][t])
            assert qc[b, t] == n and np.array_equal(qi[b, t, :n], ql[b][t]) and np.all(qi[b, t, n:st.shape[1]] == -1)
    _check_orders(bm, kc, qc, spec["mask"] == 3)


def expected_order(cnt, lists, first, documents=True):
    """Schedule order of one batch row's tiles: longest list first, ties by
    index; under a document mask, groups of tiles whose lists share their
    first (q tiles) or last (kv tiles) entry, heaviest group first (weight:
    its longest list), ties by ascending group key, and inside a group
    longest list first, ties by index.  Empty lists form one group keyed
    past every tile."""
    n, cap = lists.shape
    if not documents:
        return sorted(range(n), key=lambda t: (-int(cnt[t]), t))
    group = [int(lists[t, 0 if first else cnt[t] - 1]) if cnt[t] > 0 else cap for t in range(n)]
    weight = {}
    for t in range(n):
        weight[group[t]] = max(weight.get(group[t], 0), int(cnt[t]))
    return sorted(range(n), key=lambda t: (-weight[group[t]], group[t], -int(cnt[t]), t))


def _check_orders(bm, kc, qc, documents):
    """q_order / kv_order against the schedule order above."""
    ki, qi = bm.kv_index.cpu().numpy(), bm.q_index.cpu().numpy()
    for order, cnt, lists, first in ((bm.q_order, kc, ki, True), (bm.kv_order, qc, qi, False)):
        o = order.cpu().numpy()
        for b in range(cnt.shape[0]):
            n = cnt.shape[1]
            assert np.array_equal(o[b, :n], expected_order(cnt[b], lists[b], first, documents))


def test_doc_config_shape_mask():
    """The packed-document workload's mask (lengths uniform in [256, 4096])."""
    w = synth.WORKLOADS["doc_packed"]
    lens = synth.doc_lengths(w.S, 256, 4096, w.seed)
    ids = torch.from_numpy(synth.doc_ids_from_lengths(lens)).to(torch.int32)[None]
    bm = fa.build_block_mask(3, 1, w.S, w.S, doc_ids=dev(ids))
    torch.cuda.synchronize()
    var = oracle.Variant(mask=3, doc_ids=ids.numpy())
    # brute force on a band of query tiles (full check of every tile in them)
    st = bm.tile_state.cpu().numpy()[0]
    for qt in (0, 1, 37, 128, 200, 255):
        rows = np.arange(qt * 128, qt * 128 + 128)
        ok = oracle.allowed(var, 0, rows, np.arange(w.S))
        for kt in range(256):
            blk = ok[:, kt * 128:(kt + 1) * 128]
            want = 0 if not blk.any() else (2 if blk.all() else 1)
            assert st[qt, kt] == want, (qt, kt)


@pytest.mark.parametrize("case", [2, 4, 7])
def test_visited_with_block_mask(case):
    """With a block mask the kernel processes exactly the listed blocks:
    128/step key steps per listed block, minus steps past Skv."""
    spec, B, Sq, Skv = CASES[case]
    doc = _docs(B, Sq, 40 + case) if spec["mask"] == 3 else None
    H = 2
    q, k, v = (dev(t) for t in synth.qkv(B, H, H, Sq, Skv, 128, 1))
    bm = fa.build_block_mask(spec["mask"], B, Sq, Skv, window=spec.get("window", 0), doc_ids=dev(doc))
    nq = -(-Sq // 128)
    vis = torch.zeros((B, H, nq), dtype=torch.int32, device="cuda")
    fa.forward(q, k, v, doc_ids=dev(doc), block_mask=bm, visited=vis, **spec)
    torch.cuda.synchronize()
    step = fa.fa_fwd_kv_step(128, fa.FA_BF16)
    var = oracle.Variant(doc_ids=None if doc is None else doc.numpy(), **spec)
    _, kvl, _ = oracle.tile_states(var, B, Sq, Skv, 128, 128)
    for b in range(B):
        lists = kvl[b if spec["mask"] == 3 else 0]
        for qt in range(nq):
            want = sum(sum(1 for s0 in range(kt * 128, kt * 128 + 128, step) if s0 < Skv) for kt in lists[qt])
            for h in range(H):
                assert int(vis[b, h, qt]) == want


def _unsorted_ids(pattern, B, S, seed):
    rng = np.random.default_rng(seed)
    if pattern == "random":  # ids drawn per token from a small alphabet
        ids = rng.integers(0, 4, size=(B, S))
    else:  # 128-token blocks alternating {0 | 2} halves with blocks of id 1
        blk = np.arange(S) // 128
        ids = np.where(blk % 2 == 0, np.where(np.arange(S) % 128 < 64, 0, 2), 1)
        ids = np.broadcast_to(ids, (B, S)).copy()
        ids[:, rng.integers(0, S)] = 5  # one stray id
    return torch.from_numpy(ids.astype(np.int32))


@pytest.mark.parametrize("pattern", ["random", "interleaved"])
def test_builder_unsorted_doc_ids(pattern):
    """Document ids need not be sorted: blocks whose id ranges overlap without
    a common id must come out EMPTY, found by the pair check."""
    B, S = 2, 1100
    doc = _unsorted_ids(pattern, B, S, 90)
    bm = fa.build_block_mask(3, B, S, S, doc_ids=dev(doc))
    torch.cuda.synchronize()
    st, kvl, ql = oracle.tile_states(oracle.Variant(mask=3, doc_ids=doc.numpy()), B, S, S, 128, 128)
    assert np.array_equal(bm.tile_state.cpu().numpy(), st)
    kc, ki = bm.kv_count.cpu().numpy(), bm.kv_index.cpu().numpy()
    for b in range(B):
        for t in range(st.shape[1]):
            n = len(kvl[b][t])
            assert kc[b, t] == n and np.array_equal(ki[b, t, :n], kvl[b][t])
    _check_orders(bm, kc, bm.q_count.cpu().numpy(), True)
    if pattern == "interleaved":  # the case the id ranges alone cannot decide
        assert (st == 0).sum() > 0 and (st == 1).sum() > 0


@pytest.mark.parametrize("mask", [1, 3])
def test_orders_change_nothing_but_schedule(mask):
    """Forward and backward results are bit-identical with and without the
    schedule orders (only the workgroup-to-tile map changes)."""
    B, H, S, D = 2, 2, 900, 128
    q, k, v = (dev(t) for t in synth.qkv(B, H, H, S, S, D, 77))
    do = dev(synth.randn((B, H, S, D), 78))
    doc = _docs(B, S, 79, lo=50, hi=400) if mask == 3 else None
    res = []
    for orders in (True, False):
        bm = fa.build_block_mask(mask, B, S, S, doc_ids=dev(doc), orders=orders)
        o, lse = fa.forward(q, k, v, mask=mask, doc_ids=dev(doc), block_mask=bm, return_lse=True)
        res.append((o, lse) + tuple(fa.backward(q, k, v, o, do, lse, mask=mask, doc_ids=dev(doc), block_mask=bm)))
    torch.cuda.synchronize()
    for x, y in zip(*res):
        assert torch.equal(x, y)


def test_rebuild_into_overwrites_everything():
    """Rebuilding into an existing mask (no allocation) for other document ids
    leaves exactly what a fresh build writes: every array, including the
    unused list tails, is rewritten."""
    B, S = 2, 1500
    first = _docs(B, S, 90, lo=1, hi=60)      # many short documents: long lists
    second = _docs(B, S, 91, lo=400, hi=900)  # few long ones
    bm = fa.build_block_mask(3, B, S, S, doc_ids=dev(first))
    fa.build_block_mask(3, B, S, S, doc_ids=dev(second), into=bm)
    fresh = fa.build_block_mask(3, B, S, S, doc_ids=dev(second))
    torch.cuda.synchronize()
    for name in ("tile_state", "kv_count", "kv_index", "q_count", "q_index", "q_order", "kv_order"):
        assert torch.equal(getattr(bm, name), getattr(fresh, name)), name
