"""One query's CSA2 step from raw stored bytes, fp64 (test infrastructure only).

[架构详解 §3 mode table]: every mode computes its own query and SWA KV.
  Full    -- computes indexer Q/K and its own Top-K; also builds the pool.
  Reindex -- computes its own indexer Q and a new Top-K, re-scoring only the
             pool, against the most recent Full layer's indexer K.
  Reuse   -- no indexer; reuses the most recent Top-K indices.
[架构详解 §3.2]: the Full layer scans all visible entries, takes its own
Top-512 and builds the pool of at most 2048 blocks of 8 positions.
[架构详解 §3.1]: the encoder compresses m=2 tokens per entry (prefill
chunks), the decoder m=1.

Raw layouts (one query): q_idx uint16 [32, 128] (bf16 bits); w float [32];
k_idx uint16 [N, 128] (bf16 bits), uint8 [N, 128] (FP8 E4M3FN) or uint8
[N, 68] (MXFP4: 64 bytes of E2M1, then 4 E8M0 scales);
q uint16 [64, 512] (bf16 bits); kv_fp4 uint8 [N, 256]; kv_scale uint8
[N, 16] (E8M0); swa uint8 [S, 512] (FP8 E4M3FN), slot i holding token
swa_pos0 + i.
"""
import numpy as np

from . import formats, indexer, topk, attention as attn

CHUNK = 1 << 16


def decode_index_keys(k_raw, kdtype):
    """Indexer keys -> fp64 [N, 128].  "bf16": uint16 [N, 128] bits; "fp8":
    uint8 [N, 128] E4M3FN; "mxfp4" (the FP4 indexer QK path of [V4 essay
    §10.2]): uint8 [N, 68] rows, 64 bytes of E2M1 (OCP MXFP4 nibble order)
    then the 4 E8M0 scales of dims 32 q .. 32 q + 31; "mxfp4_qk": the same
    keys, with the query quantised too (see quantise_query)."""
    if kdtype == "bf16":
        return formats.bf16_to_f64(k_raw)
    if kdtype == "fp8":
        return formats.e4m3_to_f64(k_raw)
    if kdtype in ("mxfp4", "mxfp4_qk"):
        k_raw = np.asarray(k_raw, dtype=np.uint8)
        return formats.mxfp4_to_f64(k_raw[..., :64], k_raw[..., 64:68])
    raise ValueError(f"unknown indexer K dtype {kdtype!r}")


def quantise_query(q):
    """The query on the FP4 QK path as well ([V4 essay §10.2] puts the
    indexer's QK path, not only its keys, under FP4; the training side
    quantises to FP4 and computes with the dequantised values): each head's
    128 dims as four OCP MXFP4 blocks of 32 (formats.f64_to_mxfp4), decoded
    back to the values the products use.  fp64 [32, 128] -> fp64 [32, 128]."""
    packed, scales = formats.f64_to_mxfp4(q)
    return formats.mxfp4_to_f64(packed, scales)


def _query(q_raw, w, kdtype=None):
    q = formats.bf16_to_f64(q_raw)
    if kdtype == "mxfp4_qk":
        q = quantise_query(q)
    return q, np.asarray(w, dtype=np.float64)


def scores_prefix(q_raw, w, k_raw, kdtype, vis, chunk=CHUNK):
    """Scores of positions [0, vis), decoded and scored chunk by chunk."""
    q, wf = _query(q_raw, w, kdtype)
    out = np.empty(int(vis), dtype=np.float64)
    for lo in range(0, int(vis), chunk):
        hi = min(int(vis), lo + chunk)
        out[lo:hi] = indexer.index_scores(q, wf, decode_index_keys(k_raw[lo:hi], kdtype))
    return out


def scores_at(q_raw, w, k_raw, kdtype, positions):
    """Scores of the given positions only."""
    q, wf = _query(q_raw, w, kdtype)
    positions = np.asarray(positions, dtype=np.int64)
    return indexer.index_scores(q, wf, decode_index_keys(k_raw[positions], kdtype))


def full_layer(q_raw, w, k_raw, kdtype, vis, k_blocks=topk.MAX_POOL_BLOCKS, top_k=topk.TOP_K):
    """Full layer: scan, block maxima, pool, Top-k inside the pool.

    [架构详解 §3.2] defines the Full layer's Top-512 over every visible entry
    and builds the pool beside it.  When the pool keeps at least top_k blocks
    (or every block), the Top-k inside the pool is that global Top-k: each
    block ranked above the block of a selected position contributes its own
    maximum, a distinct position ranked above it, so fewer than top_k blocks
    rank above it.  The global Top-k is computed too and the two are asserted
    equal in that case.
    """
    s = scores_prefix(q_raw, w, k_raw, kdtype, vis)
    bm = indexer.block_max(s, vis)
    pool = topk.block_topk(bm, k_blocks)
    pos = topk.pool_positions(pool, vis)
    idx = topk.pool_topk(s[pos], pos, top_k)
    glob = topk.flat_topk(s, vis, top_k)
    if int(k_blocks) >= int(top_k) or int(k_blocks) >= bm.shape[0]:
        assert np.array_equal(idx, glob), "pool Top-k differs from the global Top-k"
    return {"scores": s, "block_max": bm, "pool": pool, "idx": idx, "global_idx": glob}


def reindex_layer(q_raw, w, k_raw, kdtype, pool, vis, top_k=topk.TOP_K):
    """Reindex layer: re-score only the Full layer's pool with this layer's query."""
    pos = topk.pool_positions(pool, vis)
    s = scores_at(q_raw, w, k_raw, kdtype, pos)
    return {"positions": pos, "scores": s, "idx": topk.pool_topk(s, pos, top_k)}


def prefill_topk(q_raw, w, k_raw, kdtype, vis, top_k=topk.TOP_K):
    """Encoder prefill (m=2): flat Top-k over every visible entry, no pool."""
    s = scores_prefix(q_raw, w, k_raw, kdtype, vis)
    return {"scores": s, "idx": topk.flat_topk(s, vis, top_k)}


def prefill_topk_bf16(q_raw, w, k_raw, kdtype, vis, top_k=topk.TOP_K):
    """The BF16-score variant ([V4 essay §10.2]: index scores kept in BF16
    instead of FP32, for a faster selector at a small loss of recall): every
    visible entry's score rounded to bf16, then the flat Top-k over those
    values (ties by position, as everywhere).  Its set is measured by recall
    against prefill_topk, not by parity."""
    s = scores_prefix(q_raw, w, k_raw, kdtype, vis)
    sb = formats.f64_to_bf16(s)
    return {"scores": s, "scores_bf16": sb,
            "idx": topk.flat_topk(formats.bf16_to_f64(sb), vis, top_k)}


def decode_main_kv(kv_fp4, kv_scale, kv_fmt="e8m0_32"):
    """Main-KV entries -> fp64: E2M1 with an E8M0 scale per 32 elements
    ("e8m0_32", OCP MXFP4) or with an E4M3 scale per 16 channels ("e4m3_16",
    the layout [架构详解 §4] describes)."""
    if kv_fmt == "e8m0_32":
        return formats.mxfp4_to_f64(kv_fp4, kv_scale)
    if kv_fmt == "e4m3_16":
        return formats.fp4e4_to_f64(kv_fp4, kv_scale)
    raise ValueError(f"unknown main-KV format {kv_fmt!r}")


def attention(q_raw, kv_fp4, kv_scale, idx, swa_raw, swa_pos0, q_pos, sm_scale,
              window=attn.WINDOW, replay_start=-1, sink=None, kv_fmt="e8m0_32"):
    """Selected main entries (idx != -1) plus the SWA window, one softmax
    (with an optional per-head sink, see attention.sparse_attention)."""
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[idx >= 0]
    main = decode_main_kv(kv_fp4[sel], kv_scale[sel], kv_fmt)
    wpos = attn.window_positions(q_pos, swa_pos0, swa_raw.shape[0], window, replay_start)
    swa = formats.e4m3_to_f64(swa_raw[wpos - int(swa_pos0)])
    entries = np.concatenate([main, swa], axis=0)
    return attn.sparse_attention(formats.bf16_to_f64(q_raw), entries, sm_scale, sink)


def kv_append(kv_fp4, kv_scale, swa, kv_new_bits, swa_new_bits, pos, swa_pos0,
              kv_fmt="e8m0_32"):
    """The KV append step ([架构详解 §4]: main KV stored as MXFP4, SWA KV as
    FP8): token i of sequence b sits at position p = pos[b] + i; its main
    entry is encoded into row p of (kv_fp4, kv_scale) when 0 <= p < N_cap
    (scales E8M0 per 32 or E4M3 per 16, by kv_fmt), and its window entry
    into row p - swa_pos0[b] of swa when that row exists.  Returns updated
    copies of the three caches (numpy uint8)."""
    encode = {"e8m0_32": formats.f64_to_mxfp4, "e4m3_16": formats.f64_to_fp4e4}[kv_fmt]
    kv_fp4, kv_scale = np.array(kv_fp4, np.uint8), np.array(kv_scale, np.uint8)
    swa = None if swa is None else np.array(swa, np.uint8)
    B, n_new = kv_new_bits.shape[0], kv_new_bits.shape[1]
    n_cap = kv_fp4.shape[1]
    for b in range(B):
        for i in range(n_new):
            p = int(pos[b]) + i
            if 0 <= p < n_cap:
                kv_fp4[b, p], kv_scale[b, p] = encode(formats.bf16_to_f64(kv_new_bits[b, i]))
            if swa_new_bits is not None:
                j = p - int(swa_pos0[b])
                if 0 <= j < swa.shape[1]:
                    swa[b, j] = formats.f64_to_e4m3(formats.bf16_to_f64(swa_new_bits[b, i]))
    return kv_fp4, kv_scale, swa


def unpage(pool, block_table, page_entries):
    """Logical view of a paged cache: [B, max_pages * page_entries, ...] from
    a pool [num_pages * page_entries, ...] and block_table [B, max_pages]
    (DeepSeek-V4 essay §7.1: compressed KV and indexer K live in a paged
    cache; entry e of sequence b is row block_table[b][e // P] * P + e % P
    of the pool).  Entries on unmapped pages (ids < 0 or >= num_pages) are
    marked False in `mapped` and their rows are zeros."""
    pool = np.asarray(pool)
    bt = np.asarray(block_table, dtype=np.int64)
    P = int(page_entries)
    num_pages = pool.shape[0] // P
    B, max_pages = bt.shape
    out = np.zeros((B, max_pages * P) + pool.shape[1:], dtype=pool.dtype)
    mapped = np.zeros((B, max_pages * P), dtype=bool)
    for b in range(B):
        for j in range(max_pages):
            page = bt[b, j]
            if 0 <= page < num_pages:
                out[b, j * P:(j + 1) * P] = pool[page * P:(page + 1) * P]
                mapped[b, j * P:(j + 1) * P] = True
    return out, mapped


def layer_mode(layer):
    """Mode of layer `layer` of the 40-layer model ([架构详解 §1]): layers
    0-19 are the causal encoder, 20-39 the decoder; only the encoder's first
    two layers are pure sliding-window attention ("swa"); its other 18 form
    three groups of six, each a Full layer then five Reuse layers; the
    decoder's 20 form five groups of four, the first Full + three Reuse, the
    other four Reindex + three Reuse.  None outside 0..39."""
    if not 0 <= layer < 40:
        return None
    if layer < 2:
        return "swa"
    if layer < 20:
        return "full" if (layer - 2) % 6 == 0 else "reuse"
    group, first = divmod(layer - 20, 4)
    if first:
        return "reuse"
    return "full" if group == 0 else "reindex"
