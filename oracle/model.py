"""Layer types of the hybrid attention stack, evaluated one query at a time (oracle side).

[chaosnode], "Hybrid Attention: CSA und HCA": CSA and HCA alternate across
layers. [golem], "Komprimierte Erinnerung für längere Kontexte": the first two
layers use only the sliding window, without compression; HCA does no
selection; CSA keeps 512 or 1,024 entries chosen by the indexer.

A layer at query position t sees: compressed entries whose block ends at or
before t (entry e of ratio m covers [e*m, e*m+m)), and the raw window
max(0, t-W+1) .. t. CSA attends over the indexer's top-k of the visible
entries plus the window; HCA over every visible entry plus the window; a
window-only layer over the window alone.

Parity: CSA with k >= n_vis equals HCA, checked in tests; the pieces are
pinned in their own modules.
"""

import numpy as np

from . import compress as C
from . import indexer as I
from . import attention as A

WINDOW = 128      # [webconsulting] "Das Wichtigste": the last 128 tokens stay uncompressed


def csa_query(q_raw, t, iq, w, ik, ent_k, ent_v, win_k, win_v, m, k, W=WINDOW,
              base=10000.0, sm_scale=None, win_first=0):
    """CSA layer for one query. ik/ent_k/ent_v dequantized [rows, .]; win_* by position.

    Returns (o [H, D], lse [H], selected ids [k], scores of the visible entries).
    """
    n_vis = I.n_visible(t, m, rows=ik.shape[0])
    scores = I.index_scores(iq, w, ik[:n_vis])
    sel = I.topk_select(scores, n_vis, k)
    o, lse = A.attend_query(q_raw, t, sel, ent_k, ent_v, win_k, win_v, W, base, sm_scale, win_first)
    return o, lse, sel, scores


def hca_query(q_raw, t, ent_k, ent_v, win_k, win_v, m, W=WINDOW, base=10000.0,
              sm_scale=None, n_entries=None, win_first=0):
    """HCA layer for one query (n_entries = 0 gives a window-only layer)."""
    n_vis = I.n_visible(t, m, rows=ent_k.shape[0])
    if n_entries is not None:
        n_vis = min(n_vis, int(n_entries))
    return A.attend_query(q_raw, t, np.arange(n_vis), ent_k, ent_v, win_k, win_v, W, base, sm_scale,
                          win_first)


def window_query(q_raw, t, win_k, win_v, W=WINDOW, base=10000.0, sm_scale=None, win_first=0):
    """Window-only layer (the first two layers of the stack)."""
    empty = np.zeros((0, win_k.shape[-1]))
    return A.attend_query(q_raw, t, np.zeros(0, np.int64), empty, empty, win_k, win_v, W, base, sm_scale,
                          win_first)


def build_caches(raw_k, raw_v, gate, pos_bias, kv_fmt, base=10000.0, raw_ik=None, ik_fmt=None):
    """Compress a whole prefix [0, T) of one layer and build its window rows.

    Returns dict with encoded stores ('ent_k', 'ent_v', 'ik', 'win_k', 'win_v'),
    each encoded store being what the kernels read, plus the dequantized float64
    views ('dk', 'dv', 'dik', 'dwk', 'dwv') the oracle attends over. Window rows
    are the m = 1 compression of every token (row p holds position p).
    """
    m = int(np.asarray(pos_bias).shape[0])
    k32, v32, ik32 = C.compress(raw_k, raw_v, gate, pos_bias, 0, base, raw_ik)
    ones = np.zeros(1, np.float32)
    wk32, wv32, _ = C.compress(raw_k, raw_v, np.zeros(np.asarray(gate).shape, np.float32), ones, 0, base)
    out = {
        'ent_k': C.encode_kv(k32, kv_fmt), 'ent_v': C.encode_kv(v32, kv_fmt),
        'win_k': C.encode_kv(wk32, kv_fmt), 'win_v': C.encode_kv(wv32, kv_fmt),
        'm': m,
    }
    out['dk'], out['dv'] = C.decode_kv(out['ent_k']), C.decode_kv(out['ent_v'])
    out['dwk'], out['dwv'] = C.decode_kv(out['win_k']), C.decode_kv(out['win_v'])
    if raw_ik is not None:
        out['ik'] = C.encode_ik(ik32, ik_fmt)
        out['dik'] = C.decode_ik(out['ik'])
    return out
