"""Attention over compressed entries plus the raw sliding window (oracle side).

[chaosnode], "Hybrid Attention: CSA und HCA": CSA attends over the top-k
compressed blocks chosen per query; HCA uses dense attention over all
compressed blocks. [webconsulting], "Das Wichtigste" and "Kompression und
Selektion": the most recent 128 tokens are always kept uncompressed in a
sliding window. [golem], "Komprimierte Erinnerung für längere Kontexte": both
mechanisms add the uncompressed last 128 tokens so that tokens not yet
compressed into a block still contribute; the first two layers use only that
window.

Readings: one joint softmax over the key list [entries] ++ [window rows];
logits sigma * (q . k) with sigma = 1/sqrt(D) unless given; the query is
rotated at its own position; the window is positions max(0, t-W+1) .. t and
includes the query's own token; an entry may cover a position also in the
window, and both are kept (no de-duplication, no attention sink).

Parity: pinned in tests against torch's scaled-dot-product attention in
float64 (m = 1 with every entry selected is dense causal attention; adding the
window equals dense attention with +ln 2 on the window keys' logits), against
sliding-window attention for window-only layers, and against a single visible
key returning its value.
"""

import numpy as np

from . import rope


def window_positions(t, W):
    return np.arange(max(0, int(t) - int(W) + 1), int(t) + 1, dtype=np.int64)


def attend(q, K, V, sm_scale):
    """q [H, D], K [L, D], V [L, D] -> (o [H, D], lse [H]); one softmax over the L keys."""
    q = np.asarray(q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    H, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1] if V.ndim == 2 else D)), np.full(H, -np.inf)
    logits = sm_scale * (q @ K.T)
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    l = p.sum(axis=-1, keepdims=True)
    o = (p @ V) / l
    return o, (mx + np.log(l))[:, 0]


def gather_keys(t, entry_ids, ent_k, ent_v, win_k, win_v, W, win_first=0):
    """Key list for a query at position t.

    entry_ids: ids into ent_k/ent_v (ids < 0 are padding and skipped);
    win_k/win_v: row i holds raw position win_first + i.
    """
    ids = np.asarray(entry_ids, np.int64)
    ids = ids[ids >= 0]
    wp = window_positions(t, W) - int(win_first)
    K = np.concatenate([np.asarray(ent_k)[ids].reshape(-1, ent_k.shape[-1]),
                        np.asarray(win_k)[wp].reshape(-1, win_k.shape[-1])], axis=0)
    V = np.concatenate([np.asarray(ent_v)[ids].reshape(-1, ent_v.shape[-1]),
                        np.asarray(win_v)[wp].reshape(-1, win_v.shape[-1])], axis=0)
    return K, V


def attend_query(q_raw, t, entry_ids, ent_k, ent_v, win_k, win_v, W, base=10000.0, sm_scale=None,
                 win_first=0):
    """One query token: q_raw [H, D] before RoPE, at position t."""
    q_raw = np.asarray(q_raw, np.float64)
    D = q_raw.shape[-1]
    sigma = 1.0 / np.sqrt(D) if not sm_scale else float(sm_scale)
    q = rope.apply(q_raw, np.int64(t), base)
    K, V = gather_keys(t, entry_ids, ent_k, ent_v, win_k, win_v, W, win_first)
    return attend(q, K, V, sigma)
