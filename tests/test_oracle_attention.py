"""Pins of the oracle's sparse attention and window (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, formats, pipeline
import synth


def _sdpa(q, kv, scale):
    # Library routine: PyTorch's scaled_dot_product_attention in float64 on CPU.
    qt = torch.from_numpy(q)[None, :, None, :]             # [1, H, 1, D]
    kt = torch.from_numpy(kv)[None, None, :, :].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=scale)
    return out[0, :, 0, :].numpy()


def _textbook(q, kv, scale):
    out = np.zeros_like(q)
    lse = np.zeros(q.shape[0])
    for h in range(q.shape[0]):
        logits = [scale * float(np.dot(q[h], kv[e])) for e in range(kv.shape[0])]
        m = max(logits)
        ws = [math.exp(x - m) for x in logits]
        z = sum(ws)
        out[h] = sum(wt * kv[e] for e, wt in enumerate(ws)) / z
        lse[h] = m + math.log(z)
    return out, lse


def test_topk_all_equals_dense_attention():
    # With every entry selected, sparse attention is dense attention over
    # concat(main entries, window).
    d = synth.make("tiny_2k", T=300)
    T = 300
    q = d["q"][0, 0].numpy().view(np.uint16)
    fp4, sc = d["kv_fp4"][0].numpy(), d["kv_scale"][0].numpy()
    swa = d["swa"][0].numpy()
    idx = np.arange(T)
    out, lse = pipeline.attention(q, fp4, sc, idx, swa, T - swa.shape[0], T - 1, synth.SM_SCALE)
    kv = np.concatenate([formats.mxfp4_to_f64(fp4, sc), formats.e4m3_to_f64(swa)])
    qf = formats.bf16_to_f64(q)
    np.testing.assert_allclose(out, _sdpa(qf, kv, synth.SM_SCALE), rtol=1e-10, atol=1e-12)
    o2, l2 = _textbook(qf[:3], kv, synth.SM_SCALE)
    np.testing.assert_allclose(out[:3], o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse[:3], l2, rtol=1e-12)


def test_lse_merge_identity():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((4, 16)); kv = rng.standard_normal((40, 16))
    o, l = attention.sparse_attention(q, kv, 0.3)
    cuts = [0, 7, 8, 29, 40]
    parts = [attention.sparse_attention(q, kv[a:b], 0.3) for a, b in zip(cuts, cuts[1:])]
    lses = np.stack([p[1] for p in parts])
    L = np.logaddexp.reduce(lses, axis=0)
    merged = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    np.testing.assert_allclose(L, l, rtol=1e-13)
    np.testing.assert_allclose(merged, o, rtol=1e-12, atol=1e-14)


def test_closed_forms():
    rng = np.random.default_rng(2)
    kv = rng.standard_normal((9, 16))
    q = np.zeros((2, 16))
    o, lse = attention.sparse_attention(q, kv, 1.0)            # equal logits -> mean
    np.testing.assert_allclose(o, np.tile(kv.mean(0), (2, 1)), rtol=1e-13)
    np.testing.assert_allclose(lse, np.log(9.0))
    q = rng.standard_normal((3, 16))
    o, _ = attention.sparse_attention(q, kv, 0.0)              # scale 0 -> mean
    np.testing.assert_allclose(o, np.tile(kv.mean(0), (3, 1)), rtol=1e-13)
    o, lse = attention.sparse_attention(q, kv[4:5], 0.7)       # one entry -> that V
    np.testing.assert_allclose(o, np.tile(kv[4], (3, 1)), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * q @ kv[4])
    perm = rng.permutation(9)                                  # order does not matter
    np.testing.assert_allclose(attention.sparse_attention(q, kv[perm], 0.7)[0],
                               attention.sparse_attention(q, kv, 0.7)[0], rtol=1e-12)
    qd = 60.0 * kv[2:3] / np.linalg.norm(kv[2])                # dominant logit -> its V
    o, _ = attention.sparse_attention(qd, kv, 1.0)
    np.testing.assert_allclose(o[0], kv[2], atol=1e-6)
    o, lse = attention.sparse_attention(q, kv[:0], 1.0)        # no entries
    assert np.all(o == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("q_pos,swa_pos0,s_cap,window,replay,expect", [
    (2047, 1920, 128, 128, -1, (1920, 2047)),   # full window, current token included
    (50, 0, 128, 128, -1, (0, 50)),             # near the start of the sequence
    (2047, 1920, 128, 128, 2000, (2000, 2047)), # replay start truncates the window
    (2047, 1990, 128, 128, -1, (1990, 2047)),   # slots before swa_pos0 do not exist
    (2047, 1920, 100, 128, -1, (1920, 2019)),   # slots beyond the stored ones do not exist
    (2047, 1920, 128, 16, -1, (2032, 2047)),    # a narrower window
])
def test_window_positions(q_pos, swa_pos0, s_cap, window, replay, expect):
    p = attention.window_positions(q_pos, swa_pos0, s_cap, window, replay)
    assert p.tolist() == list(range(expect[0], expect[1] + 1))


def test_invalid_indices_are_skipped():
    d = synth.make("tiny_2k", T=64)
    q = d["q"][0, 0].numpy().view(np.uint16)
    fp4, sc, swa = d["kv_fp4"][0].numpy(), d["kv_scale"][0].numpy(), d["swa"][0].numpy()
    a = pipeline.attention(q, fp4, sc, np.array([5, -1, 9, -1]), swa, 0, 63, 0.05)
    b = pipeline.attention(q, fp4, sc, np.array([9, 5]), swa, 0, 63, 0.05)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13)


def test_sink_matches_softmax_with_a_zero_value_slot():
    # Library routine: torch.softmax over the logits with the sink logit
    # appended as one more column; the sink's column carries no value.
    rng = np.random.default_rng(31)
    q = rng.standard_normal((6, 16)); kv = rng.standard_normal((9, 16))
    sink = np.array([-np.inf, -3.0, 0.0, 2.5, 40.0, -40.0])
    scale = 0.3
    logits = torch.from_numpy(scale * (q @ kv.T))
    full = torch.cat([logits, torch.from_numpy(sink)[:, None]], dim=1)
    p = torch.softmax(full, dim=1)[:, :-1].numpy()
    out, lse = attention.sparse_attention(q, kv, scale, sink)
    np.testing.assert_allclose(out, p @ kv, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, torch.logsumexp(full, dim=1).numpy(), rtol=1e-12)
    # No sink equals the plain attention; no entries leaves lse = sink, out 0.
    o0, l0 = attention.sparse_attention(q, kv, scale)
    o1, l1 = attention.sparse_attention(q, kv, scale, np.full(6, -np.inf))
    np.testing.assert_array_equal(o0, o1); np.testing.assert_array_equal(l0, l1)
    o2, l2 = attention.sparse_attention(q, kv[:0], scale, sink)
    assert not o2.any() and np.array_equal(l2, sink)
