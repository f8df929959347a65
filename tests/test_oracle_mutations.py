"""Planted mistakes in the oracle must fail its pins (CPU only).

Each case swaps one oracle function for a plausible wrong version, re-runs
the pin that guards it and expects that pin to fail.  Mistakes are planted
only in the oracle, on the CPU.
"""
import json
import os

import numpy as np
import pytest
import torch

from oracle import attention, formats, indexer, topk

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _pin_e4m3(decode):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.array_equal(decode(codes), lib)


def _pin_mxfp4(decode):
    with open(os.path.join(GOLD, "e2_mxfp4.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        b = np.zeros(16, np.uint8); b[0] = c["byte"]
        if not np.array_equal(decode(b, np.full(1, c["scale_code"], np.uint8))[:2], c["elements"]):
            return False
    return True


def _pin_scores(score_fn):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((32, 128)); w = rng.uniform(size=32); k = rng.standard_normal((5, 128))
    want = [sum(w[h] * max(0.0, float(np.dot(q[h], k[t]))) for h in range(32)) for t in range(5)]
    return np.allclose(score_fn(q, w, k), want, rtol=1e-12)


def _pin_e1_top4(select):
    s = np.array([4.0, 3.5, 3.0, 2.5, 2.0, 1.5, 1.0, 0.5, 0.0, 1, 2, 3, 4, 5, 6, 7])
    return select(s, np.arange(16), 4).tolist() == [0, 13, 14, 15]


def _pin_block_max(bm_fn):
    s = np.arange(21, dtype=np.float64)[::-1]
    return all(list(bm_fn(s, v)) == [max(s[8 * j:min(8 * j + 8, v)]) for j in range((v + 7) // 8)]
               for v in (1, 9, 17, 21))


def _pin_window(win_fn):
    return win_fn(2047, 1920, 128, 128, -1).tolist() == list(range(1920, 2048))


def _pin_attention(attn_fn):
    rng = np.random.default_rng(9)
    q = rng.standard_normal((3, 8)); kv = rng.standard_normal((6, 8))
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(kv)[None, None].expand(1, 3, -1, -1)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=0.4)[0, :, 0].numpy()
    return np.allclose(attn_fn(q, kv, 0.4)[0], ref, rtol=1e-10)


def _e4m3_bias8(u8):
    v = formats.E4M3_VALUES[np.asarray(u8)]
    return v / 2.0


def _mxfp4_swapped_nibbles(b, sc):
    b = np.asarray(b, np.uint8)
    swapped = ((b & 0xF) << 4) | (b >> 4)
    return formats.mxfp4_to_f64(swapped.astype(np.uint8), sc)


def _scores_no_relu(q, w, k):
    return (np.asarray(k) @ np.asarray(q).T) @ np.asarray(w)


def _scores_relu_after_sum(q, w, k):
    return np.maximum((np.asarray(k) @ np.asarray(q).T) @ np.asarray(w), 0)


def _select_high_id_wins(keys, ids, k):
    order = np.lexsort((-np.asarray(ids), -np.asarray(keys)))
    return np.sort(np.asarray(ids)[order[:k]])


def _block_max_drops_partial(s, vis):
    return indexer.block_max(s, (vis // 8) * 8) if vis >= 8 else np.zeros(0)


def _window_excludes_current(q_pos, swa_pos0, s_cap, window, replay):
    return attention.window_positions(q_pos - 1, swa_pos0, s_cap, window, replay)


def _attention_unscaled(q, kv, scale):
    return attention.sparse_attention(q, kv, 1.0)


def _pin_e4m3_encode(encode):
    x = np.concatenate([formats.E4M3_VALUES[:0x7F], (formats.E4M3_VALUES[:0x7E] +
                                                     formats.E4M3_VALUES[1:0x7F]) / 2, [500.0, -3.0]])
    lib = torch.from_numpy(np.clip(x, -448, 448).astype(np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    return np.array_equal(encode(x), lib)


def _pin_mxfp4_encode(encode):
    x = np.zeros(32)
    x[:12] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, -0.2, -0.3, -6.0, 0.26]
    p, s = encode(x)
    nib = np.empty(32, np.uint8)
    nib[0::2], nib[1::2] = p & 0xF, p >> 4
    return s.tolist() == [127] and nib[:12].tolist() == [0, 2, 2, 4, 4, 6, 6, 7, 0, 9, 15, 1]


def _e4m3_ties_up(x):
    # Ties rounded away from zero instead of to the even code.
    x = np.asarray(x, np.float64)
    up = formats.f64_to_e4m3(x)
    mag = np.minimum(np.abs(x), 448.0)
    vals = formats.E4M3_VALUES[:0x7F]
    hi = np.clip(np.searchsorted(vals, mag), 0, 0x7E)
    tie = (hi > 0) & (mag - vals[np.maximum(hi - 1, 0)] == vals[hi] - mag)
    return np.where(tie, (hi | (up & 0x80)).astype(np.uint8), up)


def _mxfp4_scale_from_ceil(x):
    # Shared exponent from ceil(log2 amax) instead of floor.
    x = np.asarray(x, np.float64)
    amax = np.abs(x.reshape(-1, 32)).max(axis=-1)
    bump = np.where((amax > 0) & (np.frexp(amax)[0] != 0.5), 1.0, 0.0)
    return formats.f64_to_mxfp4(x / np.repeat(np.ldexp(1.0, bump.astype(int)), 32))[0], \
        formats.f64_to_mxfp4(x)[1] + bump.astype(np.uint8)


MUTATIONS = [
    ("fp8 exponent bias", _pin_e4m3, formats.e4m3_to_f64, _e4m3_bias8),
    ("fp4 nibble order", _pin_mxfp4, formats.mxfp4_to_f64, _mxfp4_swapped_nibbles),
    ("ReLU dropped", _pin_scores, indexer.index_scores, _scores_no_relu),
    ("ReLU after head sum", _pin_scores, indexer.index_scores, _scores_relu_after_sum),
    ("tie-break reversed", _pin_e1_top4, topk.select, _select_high_id_wins),
    ("partial block dropped", _pin_block_max, indexer.block_max, _block_max_drops_partial),
    ("window off by one", _pin_window, attention.window_positions, _window_excludes_current),
    ("softmax scale ignored", _pin_attention, attention.sparse_attention, _attention_unscaled),
    ("fp8 encode ties away", _pin_e4m3_encode, formats.f64_to_e4m3, _e4m3_ties_up),
    ("fp4 scale from ceil", _pin_mxfp4_encode, formats.f64_to_mxfp4, _mxfp4_scale_from_ceil),
]


@pytest.mark.parametrize("name,pin,good,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_planted_mistake(name, pin, good, bad):
    assert pin(good), f"pin for {name} fails on the real oracle"
    assert not pin(bad), f"pin for {name} does not catch the planted mistake"
