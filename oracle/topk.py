"""Two-level Top-K selection, fp64 keys (test infrastructure only).

[架构详解 §3.2] (also [研究摘要 §3.2]): the first Full layer scans every
visible entry and takes its own Top-512; it aggregates indexer scores per
block of 8 positions and keeps at most 2,048 blocks, a pool of at most 16,384
candidate positions.  A Reindex layer re-scores only that pool with its own
indexer query and takes a new Top-512 ([架构详解 §3 mode table]).
[架构详解 §1 config table]: top-k 512; pool at most 2048 blocks x 8.

Readings where the pages are silent:
  * order: score descending, then position (or block id) ascending;
  * "at most 2,048 blocks": keep min(2048, number of visible blocks);
  * fewer candidates than k: keep all, pad the output with -1;
  * output lists are reported in ascending index order.
"""
import numpy as np

TOP_K = 512
MAX_POOL_BLOCKS = 2048


def select(keys, ids, k):
    """Ids of the first min(k, n) items in (key desc, id asc) order, ascending."""
    keys = np.asarray(keys, dtype=np.float64)
    ids = np.asarray(ids, dtype=np.int64)
    order = np.lexsort((ids, -keys))    # primary: -key ascending; secondary: id
    return np.sort(ids[order[: int(k)]])


def pad(ids, k):
    """Ascending ids padded with -1 to length k."""
    out = np.full(int(k), -1, dtype=np.int64)
    out[: len(ids)] = ids
    return out


def block_topk(block_maxima, k_blocks=MAX_POOL_BLOCKS):
    """Pool of block ids: top min(k_blocks, nb) blocks by maximum, ascending, -1 padded."""
    bm = np.asarray(block_maxima, dtype=np.float64)
    sel = select(bm, np.arange(bm.shape[0]), min(int(k_blocks), bm.shape[0]))
    return pad(sel, k_blocks)


def pool_positions(pool_blocks, vis, block=8):
    """Positions covered by the pool's blocks that are visible (t < vis), ascending."""
    blocks = np.asarray(pool_blocks, dtype=np.int64)
    blocks = np.sort(blocks[blocks >= 0])
    pos = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < int(vis)]


def pool_topk(scores_at, positions, top_k=TOP_K):
    """Top-k among pool candidates: scores_at[i] is the score of positions[i]."""
    return pad(select(scores_at, positions, top_k), top_k)


def flat_topk(scores, vis, top_k=TOP_K):
    """Top-k over every visible position [0, vis) with no pool."""
    s = np.asarray(scores, dtype=np.float64)[: int(vis)]
    return pad(select(s, np.arange(s.shape[0]), top_k), top_k)
