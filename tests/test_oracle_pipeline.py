"""Pins of the oracle's composition functions (oracle/pipeline.py), CPU only.

Each pin checks a pipeline function against something other than itself:
torch's own dtype casts for the key decoding, pure-Python loops for the
scores, Python's `sorted` for every selection, the inverse placement map for
the KV append, and torch's scaled_dot_product_attention over an entry list
assembled by hand for the attention step.  The pins are written as functions
of the pipeline function under test so that test_oracle_mutations.py can
plant mistakes in copies of it.
"""
import numpy as np
import pytest
import torch

from oracle import formats, pipeline
import synth


# ---------------------------------------------------------------------------
# Independent helpers (no oracle arithmetic)

_E2M1_LISTING = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                 -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]   # OCP MX v1.0 E2M1 codes


def _torch_keys(k_raw, kdtype):
    t = torch.from_numpy(np.ascontiguousarray(k_raw))
    if kdtype == "bf16":
        return t.view(torch.int16).view(torch.bfloat16).to(torch.float64).numpy()
    if kdtype == "mxfp4":
        # Nibbles (even element low) through the OCP listing, scales through
        # torch's E8M0 cast, one per 32 dims.
        nib = torch.stack([t[:, :64] & 15, t[:, :64] >> 4], dim=-1).reshape(-1, 128).long()
        vals = torch.tensor(_E2M1_LISTING, dtype=torch.float64)[nib]
        sc = t[:, 64:68].contiguous().view(torch.float8_e8m0fnu).to(torch.float64)
        return (vals * sc.repeat_interleave(32, dim=1)).numpy()
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _loop_scores(q, w, k):
    out = []
    for t in range(k.shape[0]):
        total = 0.0
        for h in range(q.shape[0]):
            dot = float(np.dot(q[h], k[t]))       # one head's dot product
            total += float(w[h]) * (dot if dot > 0.0 else 0.0)
        out.append(total)
    return np.array(out)


def _sorted_pick(keys, ids, k):
    order = sorted(range(len(ids)), key=lambda i: (-keys[i], ids[i]))
    return sorted(int(ids[i]) for i in order[:k])


def _padded(ids, k):
    return ids + [-1] * (k - len(ids))


def _inputs(seed, vis, kdtype, ties=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((32, 128))
    if ties:
        # Integer-valued keys from a few distinct rows: many exactly equal
        # scores and equal block maxima.
        base = np.round(rng.standard_normal((5, 128)) * 2)
        kf = base[rng.integers(0, 5, vis)]
        q = np.round(q * 2)
    else:
        kf = rng.standard_normal((vis, 128))
    w = rng.uniform(size=32)
    q_raw = synth.to_bf16_bits(torch.from_numpy(q).float()).numpy().view(np.uint16)
    if kdtype == "bf16":
        k_raw = synth.to_bf16_bits(torch.from_numpy(kf).float()).numpy().view(np.uint16)
    elif kdtype == "mxfp4":
        p, sc = synth.to_mxfp4(torch.from_numpy(kf).float())
        k_raw = np.concatenate([p.numpy(), sc.numpy()], axis=1)
    else:
        k_raw = synth.to_fp8_bytes(torch.from_numpy(kf).float()).numpy()
    return q_raw, w, k_raw


def _qf(q_raw):
    return torch.from_numpy(q_raw.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------------------
# Pins (each returns True when the function passed in is right)

def pin_decode_keys(fn):
    rng = np.random.default_rng(1)
    ok = True
    bf = rng.integers(0, 1 << 16, (9, 128), dtype=np.uint16)
    bf[(bf & 0x7F80) == 0x7F80] = 0x3F80                 # no inf / NaN patterns
    ok &= np.array_equal(fn(bf, "bf16"), _torch_keys(bf, "bf16"))
    f8 = rng.integers(0, 256, (9, 128), dtype=np.uint8)
    f8[(f8 & 0x7F) == 0x7F] = 0x38                       # no NaN codes
    ok &= np.array_equal(fn(f8, "fp8"), _torch_keys(f8, "fp8"))
    f4 = rng.integers(0, 256, (9, 68), dtype=np.uint8)
    f4[:, 64:] = rng.integers(100, 150, (9, 4))          # E8M0 codes away from NaN (255)
    ok &= np.array_equal(fn(f4, "mxfp4"), _torch_keys(f4, "mxfp4"))
    # A hand-made row: dims 0 and 1 in byte 0 (low nibble first), dims
    # 32..63 under the second scale.
    row = np.zeros((1, 68), np.uint8)
    row[0, 0] = 0x2F            # dim 0: code 0xF = -6; dim 1: code 0x2 = 1.0
    row[0, 16] = 0x07           # dim 32: 6.0
    row[0, 64:68] = [127, 129, 0, 127]   # 2^0, 2^2, 2^-127, 2^0
    want = np.zeros((1, 128))
    want[0, 0], want[0, 1], want[0, 32] = -6.0, 1.0, 24.0
    ok &= np.array_equal(fn(row, "mxfp4"), want)
    return bool(ok)


def pin_scores_prefix(fn):
    # Chunks of 7 over 50 positions: 7 whole chunks and a partial one.
    for kdtype in ("bf16", "fp8", "mxfp4"):
        q_raw, w, k_raw = _inputs(2, 60, kdtype)
        want = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw, kdtype))
        for vis, chunk in ((50, 7), (49, 7), (7, 7), (8, 7), (1, 3), (50, 64), (60, 1 << 16)):
            got = fn(q_raw, w, k_raw, kdtype, vis, chunk=chunk)
            if got.shape != (vis,) or not np.allclose(got, want[:vis], rtol=1e-12, atol=1e-12):
                return False
    return True


def pin_scores_at(fn):
    q_raw, w, k_raw = _inputs(3, 40, "fp8")
    pos = np.array([39, 0, 17, 17, 5])
    want = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw, "fp8")[pos])
    return np.allclose(fn(q_raw, w, k_raw, "fp8", pos), want, rtol=1e-12, atol=1e-12)


def _brute_full(q_raw, w, k_raw, kdtype, vis, kb, k):
    s = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw[:vis], kdtype))
    nb = (vis + 7) // 8
    bm = [max(s[8 * j:min(8 * j + 8, vis)]) for j in range(nb)]
    pool = _sorted_pick(bm, list(range(nb)), min(kb, nb))
    cand = [t for j in pool for t in range(8 * j, min(8 * j + 8, vis))]
    idx = _sorted_pick([s[t] for t in cand], cand, k)
    glob = _sorted_pick(list(s), list(range(vis)), k)
    return s, bm, _padded(pool, kb), _padded(idx, k), _padded(glob, k)


FULL_CASES = [  # (seed, vis, kdtype, k_blocks, top_k, ties)
    (10, 200, "bf16", 12, 9, False),
    (16, 180, "mxfp4", 10, 24, True),
    (11, 203, "fp8", 30, 16, True),
    (12, 64, "bf16", 2048, 512, False),     # every block kept, fewer than k positions
    (13, 97, "fp8", 6, 20, False),          # pool smaller than k: Top-k inside the pool only
    (14, 150, "bf16", 19, 19, True),
    (15, 1, "fp8", 4, 3, False),
]


def pin_full_layer(fn):
    for seed, vis, kdtype, kb, k, ties in FULL_CASES:
        q_raw, w, k_raw = _inputs(seed, vis + 5, kdtype, ties)
        s, bm, pool, idx, glob = _brute_full(q_raw, w, k_raw, kdtype, vis, kb, k)
        r = fn(q_raw, w, k_raw, kdtype, vis, k_blocks=kb, top_k=k)
        if not np.allclose(r["scores"], s, rtol=1e-12, atol=1e-12):
            return False
        if not np.allclose(r["block_max"], bm, rtol=1e-12, atol=1e-12):
            return False
        if r["pool"].tolist() != pool or r["idx"].tolist() != idx:
            return False
        if kb >= k and r["idx"].tolist() != glob:
            return False
    return True


def pin_reindex_layer(fn):
    for seed, vis, kdtype, ties in ((20, 180, "fp8", False), (21, 77, "bf16", True)):
        q_raw, w, k_raw = _inputs(seed, vis + 3, kdtype, ties)
        rng = np.random.default_rng(seed)
        nb = (vis + 7) // 8
        blocks = sorted(rng.choice(nb, size=min(9, nb), replace=False).tolist())
        pool = np.array(blocks + [-1] * 3)
        pos = [t for j in blocks for t in range(8 * j, min(8 * j + 8, vis))]
        s = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw, kdtype)[pos])
        want = _padded(_sorted_pick(list(s), pos, 13), 13)
        r = fn(q_raw, w, k_raw, kdtype, pool, vis, top_k=13)
        if r["idx"].tolist() != want or r["positions"].tolist() != pos:
            return False
        if not np.allclose(r["scores"], s, rtol=1e-12, atol=1e-12):
            return False
    return True


def pin_prefill_topk(fn):
    # (seed, vis, kdtype, ties, top_k); the last case keeps every visible
    # entry, so each one, the last included, must appear.
    for seed, vis, kdtype, ties, k in ((30, 90, "bf16", False, 16), (31, 41, "fp8", True, 16),
                                       (32, 20, "bf16", False, 24)):
        q_raw, w, k_raw = _inputs(seed, vis + 9, kdtype, ties)
        s = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw[:vis], kdtype))
        want = _padded(_sorted_pick(list(s), list(range(vis)), k), k)
        if fn(q_raw, w, k_raw, kdtype, vis, top_k=k)["idx"].tolist() != want:
            return False
    return True


def pin_kv_append(fn, kv_fmt="e8m0_32"):
    # Tiny caches with a sentinel fill: a row is rewritten exactly when some
    # new token maps to it (inverse map: i = p - pos[b] for cache row p,
    # window slot j holding token swa_pos0[b] + j); every other row keeps
    # the sentinel.  Encodings come from torch's FP8 cast and the torch MXFP4
    # recipe of the input generator.
    n_cap, s_cap, n_new = 6, 3, 5
    # The last sequence's first tokens fall before its window (rows -4..-1).
    pos = np.array([-1, 0, n_cap - 1, 3, 0])
    swa_pos0 = np.array([0, 2, 1, 5, 4])
    B = len(pos)
    rng = np.random.default_rng(40)
    kv_new = synth.to_bf16_bits(torch.from_numpy(rng.standard_normal((B, n_new, 512))).float())
    swa_new = synth.to_bf16_bits(torch.from_numpy(rng.standard_normal((B, n_new, 512))).float())
    nsc = 16 if kv_fmt == "e8m0_32" else 32
    quant = synth.to_mxfp4 if kv_fmt == "e8m0_32" else synth.to_fp4_e4m3
    fp4 = np.full((B, n_cap, 256), 0xAB, np.uint8)
    sc = np.full((B, n_cap, nsc), 0xCD, np.uint8)
    swa = np.full((B, s_cap, 512), 0xEF, np.uint8)
    args = (fp4, sc, swa, kv_new.numpy().view(np.uint16), swa_new.numpy().view(np.uint16), pos,
            swa_pos0)
    got_fp4, got_sc, got_swa = fn(*args) if kv_fmt == "e8m0_32" else fn(*args, kv_fmt=kv_fmt)
    kv_f = kv_new.view(torch.bfloat16).float()
    sw_f = swa_new.view(torch.bfloat16).float()
    for b in range(B):
        for p in range(n_cap):
            i = p - pos[b]
            if 0 <= i < n_new:
                wp, ws = quant(kv_f[b, i][None])
                want_p, want_s = wp[0].numpy(), ws[0].numpy()
            else:
                want_p, want_s = fp4[b, p], sc[b, p]
            if not (np.array_equal(got_fp4[b, p], want_p) and np.array_equal(got_sc[b, p], want_s)):
                return False
        for j in range(s_cap):
            i = swa_pos0[b] + j - pos[b]
            want = synth.to_fp8_bytes(sw_f[b, i]).numpy() if 0 <= i < n_new else swa[b, j]
            if not np.array_equal(got_swa[b, j], want):
                return False
    return True


def pin_attention(fn):
    # Stored window slots hold tokens 20 .. 27; the query sits at token 25
    # with a window of 4 and a replay start of 23, so it sees tokens 23..25
    # (slots 3..5).  Entries assembled by hand; SDPA in float64 is the check.
    rng = np.random.default_rng(50)
    n, s_cap, p0, qpos = 12, 8, 20, 25
    kv = rng.standard_normal((n, 512))
    fp4, sc = (t.numpy() for t in synth.to_mxfp4(torch.from_numpy(kv).float()))
    swa = synth.to_fp8_bytes(torch.from_numpy(rng.standard_normal((s_cap, 512))).float()).numpy()
    q_raw = synth.to_bf16_bits(torch.from_numpy(rng.standard_normal((4, 512))).float()).numpy()
    idx = np.array([7, -1, 2, 11, -1])
    main = torch.from_numpy(fp4[[7, 2, 11]])
    # MXFP4 decode by table lookup of the OCP values (independent of the oracle).
    table = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6],
                         dtype=torch.float64)
    nib = torch.stack([main & 15, main >> 4], dim=-1).reshape(3, 512).long()
    scale = torch.pow(2.0, torch.from_numpy(sc[[7, 2, 11]]).double() - 127).repeat_interleave(32, -1)
    ent = [table[nib] * scale]
    ent.append(torch.from_numpy(swa[[3, 4, 5]]).view(torch.float8_e4m3fn).double())
    e = torch.cat(ent)
    qf = torch.from_numpy(q_raw.view(np.int16)).view(torch.bfloat16).double()
    ref = torch.nn.functional.scaled_dot_product_attention(
        qf[None, :, None, :], e[None, None].expand(1, 4, -1, -1),
        e[None, None].expand(1, 4, -1, -1), scale=0.06)[0, :, 0].numpy()
    out, lse = fn(q_raw.view(np.uint16), fp4, sc, idx, swa, p0, qpos, 0.06, window=4,
                  replay_start=23)
    lse_ref = torch.logsumexp(0.06 * (qf @ e.T), dim=1).numpy()
    return bool(np.allclose(out, ref, rtol=1e-10, atol=1e-12)
                and np.allclose(lse, lse_ref, rtol=1e-12))


# ---------------------------------------------------------------------------

def test_decode_index_keys_matches_torch_casts():
    assert pin_decode_keys(pipeline.decode_index_keys)


def test_scores_prefix_across_chunk_boundaries():
    assert pin_scores_prefix(pipeline.scores_prefix)


def test_scores_at_given_positions():
    assert pin_scores_at(pipeline.scores_at)


def test_full_layer_against_brute_force():
    assert pin_full_layer(pipeline.full_layer)


@pytest.mark.parametrize("seed", range(4))
def test_full_layer_pool_topk_is_global_topk(seed):
    # With a pool of at least top_k blocks the Full layer's Top-k is the
    # Top-k over every visible position ([架构详解 §3.2]).
    vis = 700 + 37 * seed
    q_raw, w, k_raw = _inputs(60 + seed, vis, "fp8", ties=seed % 2 == 1)
    r = pipeline.full_layer(q_raw, w, k_raw, "fp8", vis, k_blocks=24, top_k=24)
    want = _padded(_sorted_pick(list(r["scores"]), list(range(vis)), 24), 24)
    assert r["idx"].tolist() == want and r["global_idx"].tolist() == want


def test_reindex_layer_against_brute_force():
    assert pin_reindex_layer(pipeline.reindex_layer)


def test_reindex_equals_flat_when_the_pool_covers_everything():
    # vis <= 8 k_blocks: the pool is every position, so Reindex is the flat
    # Top-k with the Reindex query (I4).
    q_raw, w, k_raw = _inputs(70, 100, "bf16")
    q2, w2, _ = _inputs(71, 100, "bf16")
    full = pipeline.full_layer(q_raw, w, k_raw, "bf16", 100)
    re = pipeline.reindex_layer(q2, w2, k_raw, "bf16", full["pool"], 100, top_k=30)
    flat = pipeline.prefill_topk(q2, w2, k_raw, "bf16", 100, top_k=30)
    assert re["idx"].tolist() == flat["idx"].tolist()


def test_prefill_topk_against_brute_force():
    assert pin_prefill_topk(pipeline.prefill_topk)


def _bf16_nearest(x):
    # The nearest bf16 value by search over torch's bf16 neighbours of the
    # binary32 cast (ties to the even pattern): independent of the oracle.
    c = torch.tensor([x], dtype=torch.float32).to(torch.bfloat16)
    bits = int(c.view(torch.int16).item()) & 0xFFFF
    cands = [b & 0xFFFF for b in (bits - 1, bits, bits + 1)]
    vals = [float(torch.tensor([b], dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
                  .to(torch.float64)) for b in cands]
    best = min(range(3), key=lambda i: (abs(vals[i] - x), cands[i] & 1))
    return vals[best]


def pin_prefill_topk_bf16(fn):
    # Brute force on the scores rounded to bf16: random keys, tie-heavy keys,
    # and a hand-made row whose fp64 order differs from its bf16 order.
    for seed, vis, kdtype, ties, k in ((33, 90, "bf16", False, 16), (34, 41, "fp8", True, 16),
                                       (35, 20, "bf16", False, 24)):
        q_raw, w, k_raw = _inputs(seed, vis + 9, kdtype, ties)
        s = _loop_scores(_qf(q_raw), w, _torch_keys(k_raw[:vis], kdtype))
        sb = [_bf16_nearest(float(v)) for v in s]
        want = _padded(_sorted_pick(sb, list(range(vis)), k), k)
        r = fn(q_raw, w, k_raw, kdtype, vis, top_k=k)
        if r["idx"].tolist() != want:
            return False
        if formats.bf16_to_f64(r["scores_bf16"]).tolist() != sb:
            return False
    # Head 0 (weight 1) reads dim 0, head 1 (weight 2^-10) dim 1: score =
    # (1 + 2^-7) + c 2^-10.  c = 1, 2, 3 round down to 1 + 2^-7 (a three-way
    # tie, so positions decide), c = 4 is a tie that goes up to 1 + 2^-6.
    c = [1.0, 3.0, 2.0, 4.0, 0.0]   # fp64 order would take positions 1 and 3
    q = np.zeros((32, 128)); q[0, 0] = 1.0; q[1, 1] = 1.0
    w = np.zeros(32, np.float32); w[0] = 1.0; w[1] = 2.0 ** -10
    kf = np.zeros((5, 128)); kf[:, 0] = 1.0 + 2.0 ** -7; kf[:, 1] = c
    q_raw = synth.to_bf16_bits(torch.from_numpy(q).float()).numpy().view(np.uint16)
    k_raw = synth.to_bf16_bits(torch.from_numpy(kf).float()).numpy().view(np.uint16)
    r = fn(q_raw, w, k_raw, "bf16", 5, top_k=2)
    return r["idx"].tolist() == [0, 3]    # bf16: 3 (up), then position 0 of the tie


def test_prefill_topk_bf16_against_brute_force():
    assert pin_prefill_topk_bf16(pipeline.prefill_topk_bf16)


def pin_scores_fp4_query(fn):
    """The FP4 QK path with the query quantised ([V4 essay §10.2], R36), on a
    hand-worked row: head 0's first 32-dim block is [1.25, 0.6875, 0.375,
    -0.3125, 0 ..., 3.0 at dim 20, 0 ...], every other dim and head 0; the
    key is [1, 2, 4, 8, 0, ...] in MXFP4 bytes written out by hand.

    The block's amax 3.0 gives the shared exponent floor(log2 3) - 2 = -1, so
    the elements are v / 0.5 rounded to E2M1 {0, .5, 1, 1.5, 2, 3, 4, 6}
    (ties to the even code): 2.5 -> 2 (a tie), 1.375 -> 1.5, 0.75 -> 1 (a
    tie), -0.625 -> -0.5, 6 -> 6; the query becomes [1, .75, .5, -.25, ...]
    and the score with weight 1 is relu(1 + 1.5 + 2 - 2) = 2.5.  Without the
    quantisation it is 1.25 + 1.375 + 1.5 - 2.5 = 1.625; with 16-element
    blocks the first half-block's exponent is -2 and the score 2.0."""
    q = np.zeros((32, 128))
    q[0, :4] = [1.25, 0.6875, 0.375, -0.3125]
    q[0, 20] = 3.0
    q_raw = formats.f64_to_bf16(q)
    w = np.zeros(32); w[0] = 1.0
    # Key block 0: amax 8 -> exponent 1 (code 128); elements 0.5, 1, 2, 4 ->
    # codes 1, 2, 4, 6, two per byte (low nibble first); blocks 1-3 are zero
    # (exponent -127, code 0).
    k = np.zeros((1, 68), dtype=np.uint8)
    k[0, 0], k[0, 1] = 0x21, 0x64
    k[0, 64] = 128
    got_qk = fn(q_raw, w, k, "mxfp4_qk", 1)
    got = fn(q_raw, w, k, "mxfp4", 1)
    return np.array_equal(got_qk, [2.5]) and np.array_equal(got, [1.625])


def test_scores_with_fp4_query_hand_worked():
    assert pin_scores_fp4_query(pipeline.scores_prefix)


def test_fp4_query_is_exact_for_representable_blocks():
    # Blocks whose values lie on the E2M1 grid times the block's own 2^X
    # (amax in [4, 8) 2^X) are left unchanged, so both key types score alike.
    rng = np.random.default_rng(31)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    X = rng.integers(-6, 4, size=(32, 4))
    vals = rng.choice(grid, size=(32, 4, 32)) * rng.choice([-1, 1], size=(32, 4, 32))
    vals[..., 0] = 6.0
    q = (vals * np.ldexp(1.0, X)[..., None]).reshape(32, 128)
    q_raw = formats.f64_to_bf16(q)
    assert np.array_equal(formats.bf16_to_f64(q_raw), q)
    assert np.array_equal(pipeline.quantise_query(q), q)
    w = rng.uniform(size=32)
    k = rng.integers(0, 256, size=(40, 68), dtype=np.uint8)
    k[:, 64:] = rng.integers(120, 134, size=(40, 4))
    assert np.array_equal(pipeline.scores_prefix(q_raw, w, k, "mxfp4_qk", 40),
                          pipeline.scores_prefix(q_raw, w, k, "mxfp4", 40))


def test_kv_append_placement_and_skip_rules():
    assert pin_kv_append(pipeline.kv_append)


def test_attention_assembles_selected_and_window_entries():
    assert pin_attention(pipeline.attention)


def test_kv_append_e4m3_layout():
    # The page's layout: 32 E4M3 scales per row, from the torch recipe.
    assert pin_kv_append(pipeline.kv_append, kv_fmt="e4m3_16")


def test_decode_main_kv_e4m3_layout():
    # E2M1 value listing times torch's float8_e4m3fn cast of the scales.
    rng = np.random.default_rng(51)
    fp4 = rng.integers(0, 256, (5, 256), dtype=np.uint8)
    sc = rng.integers(0, 0x7E, (5, 32), dtype=np.uint8)
    table = torch.tensor([0, .5, 1, 1.5, 2, 3, 4, 6, 0, -.5, -1, -1.5, -2, -3, -4, -6],
                         dtype=torch.float64)
    t = torch.from_numpy(fp4)
    nib = torch.stack([t & 15, t >> 4], dim=-1).reshape(5, 512).long()
    s = torch.from_numpy(sc).view(torch.float8_e4m3fn).double().repeat_interleave(16, -1)
    np.testing.assert_array_equal(pipeline.decode_main_kv(fp4, sc, "e4m3_16"),
                                  (table[nib] * s).numpy())


def pin_unpage(fn):
    """The logical view of a paged cache: a hand-written two-sequence example
    (rows named by value), and scattering a contiguous cache into shuffled
    pages (with spare pages) then reading it back."""
    P = 2
    pool = np.arange(5 * P * 3, dtype=np.int32).reshape(5 * P, 3)   # 5 pages of 2 rows
    bt = np.array([[3, 0, -1], [4, 7, 1]])      # page 7 is out of range: unmapped
    view, mapped = fn(pool, bt, P)
    want = np.zeros((2, 6, 3), np.int32)
    want[0, 0:2] = pool[6:8]
    want[0, 2:4] = pool[0:2]
    want[1, 0:2] = pool[8:10]
    want[1, 4:6] = pool[2:4]
    ok = np.array_equal(view, want)
    ok &= np.array_equal(mapped, np.array([[1, 1, 1, 1, 0, 0], [1, 1, 0, 0, 1, 1]], bool))
    rng = np.random.default_rng(5)
    B, max_pages, P, spare = 3, 4, 8, 5
    x = rng.integers(0, 255, size=(B, max_pages * P, 16), dtype=np.uint8)
    perm = rng.permutation(B * max_pages + spare)[:B * max_pages].reshape(B, max_pages)
    pool = np.zeros(((B * max_pages + spare) * P, 16), np.uint8)
    for b in range(B):
        for j in range(max_pages):
            pool[perm[b, j] * P:(perm[b, j] + 1) * P] = x[b, j * P:(j + 1) * P]
    view, mapped = fn(pool, perm, P)
    return bool(ok and np.array_equal(view, x) and mapped.all())


def test_unpage_logical_view():
    assert pin_unpage(pipeline.unpage)


def pin_layer_mode(fn):
    """The schedule's counts and group structure as the page states them:
    2 pure-SWA layers; encoder layers 2..19 in three groups of six, each
    Full then five Reuse; decoder layers 20..39 in five groups of four, the
    first starting with Full, the others with Reindex, three Reuse after
    each; nothing outside 0..39."""
    modes = [fn(layer) for layer in range(40)]
    enc, dec = modes[:20], modes[20:]
    ok = enc[:2] == ["swa", "swa"]
    ok &= all(enc[2 + 6 * g:8 + 6 * g] == ["full"] + ["reuse"] * 5 for g in range(3))
    ok &= dec[0:4] == ["full", "reuse", "reuse", "reuse"]
    ok &= all(dec[4 * g:4 * g + 4] == ["reindex", "reuse", "reuse", "reuse"] for g in range(1, 5))
    ok &= (modes.count("full"), modes.count("reindex"), modes.count("reuse"),
           modes.count("swa")) == (4, 4, 30, 2)
    ok &= fn(-1) is None and fn(40) is None
    return bool(ok)


def test_layer_schedule():
    assert pin_layer_mode(pipeline.layer_mode)
