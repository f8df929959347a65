"""Pins of the oracle's indexer score and block maximum (CPU only)."""
import json
import os

import numpy as np

from oracle import indexer, topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _e1():
    with open(os.path.join(GOLD, "e1_indexer.json")) as f:
        g = json.load(f)
    q = np.zeros((32, 128)); q[0, 0] = 1.0; q[1, 0] = -1.0
    w = np.zeros(32); w[0] = 1.0; w[1] = 0.5
    k = np.zeros((16, 128)); k[:, 0] = np.arange(16) - 8.0
    return g, q, w, k


def test_e1_hand_worked():
    g, q, w, k = _e1()
    s = indexer.index_scores(q, w, k)
    np.testing.assert_array_equal(s, g["scores"])
    np.testing.assert_array_equal(indexer.block_max(s, 16), g["block_max"])
    np.testing.assert_array_equal(topk.select(s, np.arange(16), 3), g["top3"])
    np.testing.assert_array_equal(topk.select(s, np.arange(16), 4), g["top4"])
    np.testing.assert_array_equal(topk.select(np.ones(16), np.arange(16), 5), g["all_equal_top5"])


def _brute_scores(q, w, k):
    out = []
    for t in range(k.shape[0]):
        total = 0.0
        for h in range(q.shape[0]):
            dot = 0.0
            for d in range(q.shape[1]):
                dot += q[h, d] * k[t, d]
            total += w[h] * (dot if dot > 0 else 0.0)
        out.append(total)
    return np.array(out)


def test_scores_against_loops():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((32, 128)); w = rng.uniform(size=32); k = rng.standard_normal((5, 128))
    np.testing.assert_allclose(indexer.index_scores(q, w, k), _brute_scores(q, w, k), rtol=1e-12, atol=1e-12)


def test_one_hot_weight_selects_relu_of_one_head():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((32, 128)); k = rng.standard_normal((50, 128))
    for h in (0, 17, 31):
        w = np.zeros(32); w[h] = 1.0
        np.testing.assert_allclose(indexer.index_scores(q, w, k), np.maximum(k @ q[h], 0), rtol=1e-13, atol=1e-13)


def test_positive_scaling_scales_scores_and_keeps_selection():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((32, 128)); w = rng.uniform(size=32); k = rng.standard_normal((300, 128))
    s = indexer.index_scores(q, w, k)
    np.testing.assert_allclose(indexer.index_scores(q, 4.0 * w, k), 4.0 * s, rtol=1e-13)
    np.testing.assert_allclose(indexer.index_scores(2.0 * q, w, k), 2.0 * s, rtol=1e-13)
    ids = np.arange(300)
    np.testing.assert_array_equal(topk.select(4.0 * s, ids, 20), topk.select(s, ids, 20))
    # A negative head weight would flip signs: scores are not >= 0 then.
    assert np.all(s >= 0)


def test_block_max_partial_last_block():
    s = np.arange(21, dtype=np.float64)[::-1]   # 20, 19, ..., 0
    for vis in (1, 7, 8, 9, 16, 17, 21):
        bm = indexer.block_max(s, vis)
        assert len(bm) == (vis + 7) // 8
        for j in range(len(bm)):
            assert bm[j] == max(s[t] for t in range(8 * j, min(8 * j + 8, vis)))
