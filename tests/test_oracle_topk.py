"""Pins of the oracle's two-level Top-K (CPU only)."""
import numpy as np
import pytest

from oracle import indexer, topk


def _brute(keys, k):
    order = sorted(range(len(keys)), key=lambda t: (-keys[t], t))
    return sorted(order[:k])


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_sorted_and_properties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 400))
    keys = np.round(rng.standard_normal(n) * 3) / 3      # many exact ties
    k = int(rng.integers(1, 600))
    sel = topk.select(keys, np.arange(n), k)
    assert sel.tolist() == _brute(keys.tolist(), k)
    assert len(sel) == min(k, n) and len(set(sel.tolist())) == len(sel)
    assert np.all(np.diff(sel) > 0)
    rest = np.setdiff1d(np.arange(n), sel)
    if len(rest) and len(sel):
        assert keys[sel].min() >= keys[rest].max()


def test_padding_when_fewer_candidates():
    out = topk.flat_topk(np.array([3.0, 1.0, 2.0]), 3, 5)
    assert out.tolist() == [0, 1, 2, -1, -1]
    pool = topk.block_topk(np.array([1.0, 5.0]), 4)
    assert pool.tolist() == [0, 1, -1, -1]


def _full_and_global(s, vis, kb, k):
    bm = indexer.block_max(s, vis)
    pool = topk.block_topk(bm, kb)
    pos = topk.pool_positions(pool, vis)
    return topk.pool_topk(s[pos], pos, k), topk.flat_topk(s, vis, k)


@pytest.mark.parametrize("seed", range(12))
def test_hierarchy_invariant_pool_topk_equals_global(seed):
    # With kb >= k and the same tie order, Top-k inside the pool equals the
    # global Top-k: each block ranked above the block of a top-k position
    # contributes its own maximum, a distinct position ranked above it.
    rng = np.random.default_rng(100 + seed)
    vis = int(rng.integers(1, 3000))
    kind = seed % 3
    if kind == 0:
        s = rng.standard_normal(vis)
    elif kind == 1:
        s = np.round(rng.standard_normal(vis))          # heavy ties
    else:
        s = np.full(vis, 2.5)                           # all equal
    k = int(rng.integers(1, 70))
    kb = int(rng.integers(k, k + 40))
    pool_sel, glob = _full_and_global(s, vis, kb, k)
    np.testing.assert_array_equal(pool_sel, glob)


def test_hierarchy_fails_when_pool_smaller_than_k():
    # Sanity of the invariant's premise: with kb < k/8 the pool cannot hold k.
    s = np.arange(200, dtype=np.float64)
    pool_sel, glob = _full_and_global(s, 200, 2, 30)
    assert (pool_sel >= 0).sum() == 16 and not np.array_equal(pool_sel, glob)


def test_pool_positions_clip_to_visible():
    pos = topk.pool_positions(np.array([2, 0, -1]), 20)
    assert pos.tolist() == list(range(0, 8)) + list(range(16, 20))


@pytest.mark.parametrize("seed", range(4))
def test_reindex_equals_flat_when_pool_covers_all(seed):
    rng = np.random.default_rng(200 + seed)
    vis = int(rng.integers(1, 800))
    s_full = rng.standard_normal(vis)
    s_re = rng.standard_normal(vis)
    pool = topk.block_topk(indexer.block_max(s_full, vis), 2048)   # vis <= 8*2048: all blocks
    pos = topk.pool_positions(pool, vis)
    np.testing.assert_array_equal(pos, np.arange(vis))
    np.testing.assert_array_equal(topk.pool_topk(s_re[pos], pos, 64), topk.flat_topk(s_re, vis, 64))
