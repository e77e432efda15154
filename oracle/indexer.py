"""Lightning-indexer scoring and top-k selection (oracle side).

[webconsulting], "Kompression und Selektion": the indexer scans the compressed
entries at lower numerical precision and forwards the most relevant 1,024 to the
CSA layers. [chaosnode], "Hybrid Attention: CSA und HCA": the indexer picks the
top-k compressed blocks per query and runs in FP4. [golem], "Komprimierte
Erinnerung für längere Kontexte": CSA uses 512 (Flash) or 1,024 (Pro) entries,
the indexer is a learned model, and HCA does no selection.

Reading of the score (the pages give no formula; PARITY OF THE FORMULA IS
UNPINNED by the pages, only its implementation is pinned): per query t, with
H_I indexer heads q_{t,h}, per-head weights w_{t,h} and one indexer key u_e per
compressed entry,

    I_{t,e} = sum_h w_{t,h} * max(0, q_{t,h} . u_e).

Non-finite values: max(0, x) is the IEEE 754-2019 maximum operation, which
propagates NaN (as numpy's maximum and torch's relu do): a NaN dot product of
any head makes the entry's score NaN. The pages say nothing about non-finite
inputs; propagation is the plain arithmetic reading, so nothing is dropped
silently.

Selection: among the entries visible to t (entry e covers positions
[e*m, e*m+m) and is visible when e*m + m - 1 <= t), keep the min(k, n_vis) with
the largest score; equal scores go to the lower entry index. Scores are
compared as float32 values (the precision the kernel decides in); -0 equals
+0 and NaN ranks below every number. The result is a set, returned ascending
and padded with -1 to length k.

Parity: pinned in tests against a pure-Python double loop, exact rational dot
products of MXFP4 operands, hand-derived selections with NaN key blocks and
NaN query heads, and a stable brute-force sort (ties, -0, NaN) for both the
selection and the k-th score.
"""

import numpy as np


def n_visible(t, m, rows=None):
    n = (int(t) + 1) // int(m)
    return n if rows is None else min(n, int(rows))


def index_scores(iq, w, keys):
    """iq [H, dI], w [H], keys [N, dI] (dequantized) -> scores [N] float64."""
    iq = np.asarray(iq, np.float64)
    keys = np.asarray(keys, np.float64)
    dots = keys @ iq.T                           # [N, H]
    # max(0, x) propagating NaN (IEEE 754-2019 maximum)
    return np.maximum(dots, 0.0) @ np.asarray(w, np.float32).astype(np.float64)


def topk_select(scores, n_vis, k):
    """scores [>= n_vis] -> int32 [k]: selected entry ids ascending, -1 padded."""
    s = np.asarray(scores, np.float64)[:n_vis].astype(np.float32).astype(np.float64)
    nan = np.isnan(s)
    neg = np.where(nan, 0.0, -s)
    idx = np.arange(n_vis)
    order = np.lexsort((idx, neg, nan))          # last key is the primary one
    sel = np.sort(order[:min(k, n_vis)])
    out = np.full(k, -1, np.int32)
    out[:sel.size] = sel
    return out


def kth_score(scores, n_vis, k):
    """float32 value of the k-th best visible score (the boundary of the tie band).

    The score of the min(k, n_vis)-th entry in selection order. NaN ranks below
    every number, so when that entry's score is NaN the boundary is -inf.
    """
    s = np.asarray(scores, np.float64)[:n_vis].astype(np.float32).astype(np.float64)
    s = np.where(np.isnan(s), -np.inf, s)
    if n_vis == 0:
        return np.nan
    kk = min(k, n_vis)
    return np.sort(s)[::-1][kk - 1]
