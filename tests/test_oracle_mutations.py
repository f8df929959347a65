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

from oracle import attention, formats, indexer, pipeline, topk
import test_oracle_formats as tf
import test_oracle_pipeline as pp

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


def _pin_fp4e4(decode):
    with open(os.path.join(GOLD, "e5_fp4_e4m3.json")) as f:
        cases = json.load(f)["decode"]
    for c in cases:
        b = np.zeros(16, np.uint8); b[0] = c["byte"]
        if not np.array_equal(decode(b, np.full(2, c["scale_code"], np.uint8))[:2], c["elements"]):
            return False
    # one scale per 16 elements: element 16 takes the second scale
    b = np.full(16, 0x22, np.uint8)
    v = decode(b, np.array([0x38, 0x40], np.uint8))
    return bool(np.all(v[:16] == 1.0) and np.all(v[16:] == 2.0))


def _fp4e4_scale_per_32(b, sc):
    sc = np.asarray(sc, np.uint8)
    return formats.fp4e4_to_f64(b, np.repeat(sc[..., ::2], 2, axis=-1))


def _pin_fp4e4_encode(encode):
    with open(os.path.join(GOLD, "e5_fp4_e4m3.json")) as f:
        g = json.load(f)["encode"]
    p, s = encode(np.array(g["block"], np.float64))
    nib = np.empty(16, np.uint8)
    nib[0::2], nib[1::2] = p & 0xF, p >> 4
    return s.tolist() == [g["scale_code"]] and nib.tolist() == g["nibbles"]


def _fp4e4_scale_amax_over_4(x):
    # Scale chosen for E2M1's top binade (amax / 4) instead of its maximum 6.
    return formats.f64_to_fp4e4(np.asarray(x, np.float64) * 1.5)


# Planted mistakes in copies of the pipeline's composition functions.

def _scores_prefix_tail_dropped(q_raw, w, k_raw, kdtype, vis, chunk=pipeline.CHUNK):
    q, wf = formats.bf16_to_f64(q_raw), np.asarray(w, np.float64)
    out = np.zeros(int(vis))
    for lo in range(0, int(vis) - chunk + 1, chunk):     # the partial last chunk is never scored
        out[lo:lo + chunk] = indexer.index_scores(
            q, wf, pipeline.decode_index_keys(k_raw[lo:lo + chunk], kdtype))
    return out


def _scores_prefix_shifted(q_raw, w, k_raw, kdtype, vis, chunk=pipeline.CHUNK):
    q, wf = formats.bf16_to_f64(q_raw), np.asarray(w, np.float64)
    out = np.empty(int(vis))
    for lo in range(0, int(vis), chunk):
        hi = min(int(vis), lo + chunk)
        src = k_raw[lo + (lo > 0):hi + (lo > 0)]           # chunks after the first read one row late
        out[lo:hi] = indexer.index_scores(q, wf, pipeline.decode_index_keys(src, kdtype))
    return out


def _full_layer_global_not_pool(q_raw, w, k_raw, kdtype, vis, k_blocks=2048, top_k=512):
    s = pipeline.scores_prefix(q_raw, w, k_raw, kdtype, vis)
    bm = indexer.block_max(s, vis)
    return {"scores": s, "block_max": bm, "pool": topk.block_topk(bm, k_blocks),
            "idx": topk.flat_topk(s, vis, top_k)}       # Top-k taken outside the pool


def _full_layer_pool_of_top_k(q_raw, w, k_raw, kdtype, vis, k_blocks=2048, top_k=512):
    s = pipeline.scores_prefix(q_raw, w, k_raw, kdtype, vis)
    bm = indexer.block_max(s, vis)
    pool = topk.block_topk(bm, min(k_blocks, top_k))     # pool sized by top_k
    pool = topk.pad(pool[pool >= 0], k_blocks)
    pos = topk.pool_positions(pool, vis)
    return {"scores": s, "block_max": bm, "pool": pool, "idx": topk.pool_topk(s[pos], pos, top_k)}


def _reindex_block_ids_as_positions(q_raw, w, k_raw, kdtype, pool, vis, top_k=512):
    blocks = np.sort(np.asarray(pool)[np.asarray(pool) >= 0])   # the x8 expansion forgotten
    s = pipeline.scores_at(q_raw, w, k_raw, kdtype, blocks)
    return {"positions": blocks, "scores": s, "idx": topk.pool_topk(s, blocks, top_k)}


def _reindex_unclipped(q_raw, w, k_raw, kdtype, pool, vis, top_k=512):
    blocks = np.sort(np.asarray(pool)[np.asarray(pool) >= 0])
    pos = (blocks[:, None] * 8 + np.arange(8)[None, :]).reshape(-1)
    pos = pos[pos < k_raw.shape[0]]                      # clipped to the cache, not to vis
    s = pipeline.scores_at(q_raw, w, k_raw, kdtype, pos)
    return {"positions": pos, "scores": s, "idx": topk.pool_topk(s, pos, top_k)}


def _prefill_last_entry_hidden(q_raw, w, k_raw, kdtype, vis, top_k=512):
    return pipeline.prefill_topk(q_raw, w, k_raw, kdtype, vis - 1, top_k)


def _kv_append_variant(window_shift=0, wrap_main=False, wrap_window=False):
    def fn(kv_fp4, kv_scale, swa, kv_new_bits, swa_new_bits, pos, swa_pos0):
        kv_fp4, kv_scale, swa = np.array(kv_fp4), np.array(kv_scale), np.array(swa)
        n_cap, s_cap = kv_fp4.shape[1], swa.shape[1]
        for b in range(kv_new_bits.shape[0]):
            for i in range(kv_new_bits.shape[1]):
                p = int(pos[b]) + i
                if (-n_cap <= p < n_cap) if wrap_main else (0 <= p < n_cap):
                    kv_fp4[b, p], kv_scale[b, p] = formats.f64_to_mxfp4(
                        formats.bf16_to_f64(kv_new_bits[b, i]))
                j = p - int(swa_pos0[b]) + window_shift
                if (-s_cap <= j < s_cap) if wrap_window else (0 <= j < s_cap):
                    swa[b, j] = formats.f64_to_e4m3(formats.bf16_to_f64(swa_new_bits[b, i]))
        return kv_fp4, kv_scale, swa
    return fn


def _layer_mode_variant():
    # Mistake: decoder groups of five layers (the encoder's grouping habit).
    def layer_mode(layer):
        if not 0 <= layer < 40:
            return None
        if layer < 2:
            return "swa"
        if layer < 20:
            return "full" if (layer - 2) % 6 == 0 else "reuse"
        group, first = divmod(layer - 20, 5)
        if first:
            return "reuse"
        return "full" if group == 0 else "reindex"
    return layer_mode


def _mxfp4_keys_scales_swapped(k_raw, kdtype):
    # Mistake: the MXFP4 key row's scales read in reverse order.
    if kdtype == "mxfp4":
        k_raw = np.asarray(k_raw, dtype=np.uint8)
        return formats.mxfp4_to_f64(k_raw[..., :64], k_raw[..., 64:68][..., ::-1])
    return pipeline.decode_index_keys(k_raw, kdtype)


def _unpage_variant():
    # Mistake: page j of a sequence read from pool row j * P instead of its
    # table entry's page (the table ignored).
    def unpage(pool, block_table, page_entries):
        pool = np.asarray(pool)
        bt = np.asarray(block_table)
        P = int(page_entries)
        B, max_pages = bt.shape
        out = np.zeros((B, max_pages * P) + pool.shape[1:], dtype=pool.dtype)
        for b in range(B):
            for j in range(max_pages):
                if (j + 1) * P <= pool.shape[0]:
                    out[b, j * P:(j + 1) * P] = pool[j * P:(j + 1) * P]
        return out, np.ones((B, max_pages * P), bool)
    return unpage


def _attention_variant(slot_shift=0, keep_empty=False):
    def fn(q_raw, kv_fp4, kv_scale, idx, swa_raw, swa_pos0, q_pos, sm_scale, window=128,
           replay_start=-1, sink=None):
        idx = np.asarray(idx, dtype=np.int64)
        sel = idx if keep_empty else idx[idx >= 0]
        main = formats.mxfp4_to_f64(kv_fp4[sel], kv_scale[sel])
        wpos = attention.window_positions(q_pos, swa_pos0, swa_raw.shape[0], window, replay_start)
        swa = formats.e4m3_to_f64(swa_raw[wpos - int(swa_pos0) + slot_shift])
        return attention.sparse_attention(formats.bf16_to_f64(q_raw),
                                          np.concatenate([main, swa]), sm_scale, sink)
    return fn


def _bf16_truncated(x):
    x = np.asarray(x, dtype=np.float64)
    return (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    mag = np.abs(x)
    _, e = np.frexp(np.where(mag > 0, mag, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e - 1, -126) - 7)
    r = np.floor(mag / quantum + 0.5) * quantum
    r = np.where(r > (2.0 - 2.0 ** -7) * 2.0 ** 127, np.inf, r)
    r = np.where(np.signbit(x), -r, r)
    with np.errstate(over="ignore"):
        return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bf16_through_binary32(x):
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    return formats.f64_to_bf16(x32.astype(np.float64))


def _prefill_bf16_selects_fp64(q_raw, w, k_raw, kdtype, vis, top_k=512):
    r = pipeline.prefill_topk_bf16(q_raw, w, k_raw, kdtype, vis, top_k)
    r["idx"] = topk.flat_topk(r["scores"], vis, top_k)
    return r


def _scores_query_unquantised(q_raw, w, k_raw, kdtype, vis, chunk=pipeline.CHUNK):
    # Mistake: the FP4 QK path quantises the keys only.
    return pipeline.scores_prefix(q_raw, w, k_raw, "mxfp4" if kdtype == "mxfp4_qk" else kdtype,
                                  vis, chunk)


def _scores_query_blocks_of_16(q_raw, w, k_raw, kdtype, vis, chunk=pipeline.CHUNK):
    # Mistake: the query quantised in blocks of 16 dims instead of 32.
    if kdtype != "mxfp4_qk":
        return pipeline.scores_prefix(q_raw, w, k_raw, kdtype, vis, chunk)
    q = formats.bf16_to_f64(q_raw).reshape(32, 8, 16)
    amax = np.abs(q).max(axis=-1)
    _, e = np.frexp(amax)
    X = np.where(amax > 0, np.clip(e - 3, -127, 127), -127)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    scaled = np.minimum(np.abs(q) / np.ldexp(1.0, X)[..., None], 6.0)
    near = grid[np.abs(scaled[..., None] - grid).argmin(axis=-1)]
    q4 = (np.sign(q) * near * np.ldexp(1.0, X)[..., None]).reshape(32, 128)
    return indexer.index_scores(q4, np.asarray(w, np.float64),
                                pipeline.decode_index_keys(k_raw[:vis], "mxfp4"))


MUTATIONS = [
    ("bf16 scores truncated", tf.pin_bf16_encode, formats.f64_to_bf16, _bf16_truncated),
    ("bf16 scores ties away", tf.pin_bf16_encode, formats.f64_to_bf16, _bf16_ties_away),
    ("bf16 scores rounded twice", tf.pin_bf16_encode, formats.f64_to_bf16, _bf16_through_binary32),
    ("bf16 Top-k on fp64 scores", pp.pin_prefill_topk_bf16, pipeline.prefill_topk_bf16,
     _prefill_bf16_selects_fp64),
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
    ("fp4/e4m3 scale per 32", _pin_fp4e4, formats.fp4e4_to_f64, _fp4e4_scale_per_32),
    ("fp4/e4m3 scale from amax / 4", _pin_fp4e4_encode, formats.f64_to_fp4e4,
     _fp4e4_scale_amax_over_4),
    ("score chunk tail dropped", pp.pin_scores_prefix, pipeline.scores_prefix,
     _scores_prefix_tail_dropped),
    ("score chunk slice off by one", pp.pin_scores_prefix, pipeline.scores_prefix,
     _scores_prefix_shifted),
    ("full Top-k outside the pool", pp.pin_full_layer, pipeline.full_layer,
     _full_layer_global_not_pool),
    ("pool sized by top_k", pp.pin_full_layer, pipeline.full_layer, _full_layer_pool_of_top_k),
    ("reindex block ids as positions", pp.pin_reindex_layer, pipeline.reindex_layer,
     _reindex_block_ids_as_positions),
    ("reindex pool not clipped to vis", pp.pin_reindex_layer, pipeline.reindex_layer,
     _reindex_unclipped),
    ("prefill last entry hidden", pp.pin_prefill_topk, pipeline.prefill_topk,
     _prefill_last_entry_hidden),
    ("append window row off by one", pp.pin_kv_append, pipeline.kv_append,
     _kv_append_variant(window_shift=1)),
    ("append main skip rule dropped", pp.pin_kv_append, pipeline.kv_append,
     _kv_append_variant(wrap_main=True)),
    ("append window skip rule dropped", pp.pin_kv_append, pipeline.kv_append,
     _kv_append_variant(wrap_window=True)),
    ("attention window slot off by one", pp.pin_attention, pipeline.attention,
     _attention_variant(slot_shift=-1)),
    ("attention empty slots kept", pp.pin_attention, pipeline.attention,
     _attention_variant(keep_empty=True)),
    ("mxfp4 key scales reversed", pp.pin_decode_keys, pipeline.decode_index_keys,
     _mxfp4_keys_scales_swapped),
    ("unpage with the page index as the row offset", pp.pin_unpage, pipeline.unpage,
     _unpage_variant()),
    ("schedule with decoder groups of five", pp.pin_layer_mode, pipeline.layer_mode,
     _layer_mode_variant()),
    ("fp4 QK path with the query left in bf16", pp.pin_scores_fp4_query, pipeline.scores_prefix,
     _scores_query_unquantised),
    ("fp4 query in blocks of 16", pp.pin_scores_fp4_query, pipeline.scores_prefix,
     _scores_query_blocks_of_16),
]


def _holds(pin, fn):
    # A pin that raises on a wrong function has caught it as well.
    try:
        return bool(pin(fn))
    except (AssertionError, IndexError, ValueError):
        return False


@pytest.mark.parametrize("name,pin,good,bad", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pin_catches_planted_mistake(name, pin, good, bad):
    assert pin(good), f"pin for {name} fails on the real oracle"
    assert not _holds(pin, bad), f"pin for {name} does not catch the planted mistake"
