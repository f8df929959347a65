"""Indexer score and block maximum, fp64 (test infrastructure only).

[V4 essay §3.2]: the Lightning Indexer projects the query into a small
indexer space and matches it against compressed index keys, one score per
entry.  [架构详解 §1 config table]: 32 indexer heads of 128 dims.
[架构详解 §3.2]: indexer K is projected from main KV, so one 128-dim key per
entry is shared by all heads.  The pages print no formula; the reading taken
is the per-head ReLU-weighted sum

    s_t = sum_{h<32} w_h * max(0, sum_{d<128} qI[h, d] * KI[t, d]).

[架构详解 §3.2]: the Full layer also aggregates indexer scores per block of 8
positions; the aggregation operator is unstated and is read as the maximum
over the block's visible positions, with block j = positions [8j, 8j+8).
"""
import numpy as np

BLOCK = 8


def index_scores(q_idx, w, k_idx):
    """q_idx [32, 128], w [32], k_idx [T, 128] (all fp64) -> scores [T]."""
    q_idx = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    k_idx = np.asarray(k_idx, dtype=np.float64)
    logits = k_idx @ q_idx.T            # [T, 32]: q_h . k_t for every head
    return np.maximum(logits, 0.0) @ w  # ReLU, then the w-weighted head sum


def num_blocks(vis, block=BLOCK):
    """Number of (possibly partial) blocks that cover [0, vis)."""
    return (int(vis) + block - 1) // block


def block_max(scores, vis, block=BLOCK):
    """Maximum score of each block over its visible positions t < vis."""
    s = np.asarray(scores, dtype=np.float64)[: int(vis)]
    nb = num_blocks(vis, block)
    padded = np.full(nb * block, -np.inf)
    padded[: s.shape[0]] = s
    return padded.reshape(nb, block).max(axis=1)
