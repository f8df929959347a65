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
the current token, no norm or rotary inside.  An attention sink is optional
(sparse_attention's `sink`; none by default).
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


def sparse_attention(q, entries, sm_scale, sink=None):
    """Softmax attention of q [H, D] over entries [E, D] used as K and V.

    Returns (out [H, D], lse [H]) with lse the natural-log normaliser
    log sum_e exp(sm_scale * q_h . k_e).  With no entries: out 0, lse -inf.

    sink: None, or [H] per-head sink logits (DeepSeek-V4 essay §4.3: each
    head may put part of its probability mass on a virtual sink instead of
    the history).  The sink adds exp(sink_h) to head h's normaliser and
    contributes no value; -inf is no sink.
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(entries, dtype=np.float64)
    logits = float(sm_scale) * (q @ kv.T)          # [H, E]
    s = (np.full(q.shape[0], -np.inf) if sink is None
         else np.asarray(sink, dtype=np.float64).reshape(q.shape[0]))
    mu = np.maximum(logits.max(axis=1) if kv.shape[0] else np.full(q.shape[0], -np.inf), s)
    if kv.shape[0] == 0 and np.all(np.isneginf(mu)):
        return np.zeros_like(q), np.full(q.shape[0], -np.inf)
    safe = np.where(np.isneginf(mu), 0.0, mu)      # heads with nothing at all: l = 0
    p = np.exp(logits - safe[:, None])
    l = p.sum(axis=1) + np.exp(s - safe)
    with np.errstate(invalid="ignore", divide="ignore"):
        out = np.where(l[:, None] > 0, (p @ kv) / np.where(l > 0, l, 1.0)[:, None], 0.0)
        lse = np.where(l > 0, safe + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return out, lse
