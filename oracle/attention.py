"""Sparse multi-query attention with the SWA window, fp64 (test infrastructure only).

[架构详解 §1 config table]: 64 query heads of 512 dims; SWA window 128.
[架构详解 §3.2 / §9 step 5]: decode attends to the CSA2-selected global KV
plus this layer's own SWA KV.  [V4 essay §4.3]: a compressed KV entry serves
as both key and value.  [V4 essay §3.3]: the window keeps the most recent 128
uncompressed tokens.  [架构详解 §5]: a replayed window is truncated to
[max(s, i-W+1), i] for replay start s.

Readings: one softmax over the union of selected main entries and window
tokens (no de-duplication), each entry used as both K and V, logits scaled by
sm_scale (1/sqrt(512) in the workloads), window [q_pos-W+1, q_pos] including
the current token, no attention sink, no norm or rotary inside.
"""
import numpy as np

WINDOW = 128


def window_positions(q_pos, swa_pos0, s_cap, window=WINDOW, replay_start=-1):
    """Token positions of the SWA window for a query at q_pos.

    Slot p - swa_pos0 of the stored window holds token p; a position is used
    only when that slot exists (0 <= p - swa_pos0 < s_cap).
    """
    lo = max(int(q_pos) - int(window) + 1, int(swa_pos0), 0)
    if replay_start is not None and int(replay_start) >= 0:
        lo = max(lo, int(replay_start))
    hi = min(int(q_pos), int(swa_pos0) + int(s_cap) - 1)
    return np.arange(lo, hi + 1, dtype=np.int64) if hi >= lo else np.zeros(0, np.int64)


def sparse_attention(q, entries, sm_scale):
    """Softmax attention of q [H, D] over entries [E, D] used as K and V.

    Returns (out [H, D], lse [H]) with lse the natural-log normaliser
    log sum_e exp(sm_scale * q_h . k_e).  With no entries: out 0, lse -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(entries, dtype=np.float64)
    if kv.shape[0] == 0:
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    logits = float(sm_scale) * (q @ kv.T)          # [H, E]
    mu = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mu)
    l = p.sum(axis=1)
    out = (p @ kv) / l[:, None]
    lse = mu[:, 0] + np.log(l)
    return out, lse
