"""KV compression by softmax-gated pooling with a learned positional bias (oracle side).

[chaosnode], "Hybrid Attention: CSA und HCA": CSA compresses KV entries 4x
along the sequence by softmax-gated pooling with a learned positional bias;
HCA compresses 128x. [webconsulting], "Kompression und Selektion": HCA merges
each 128 tokens into one entry through learned weightings, CSA groups 4 tokens.
[golem], "Komprimierte Erinnerung für längere Kontexte": several token
embeddings are merged into one value (4 for CSA, 128 for HCA).

Readings (the pages give no formula):

* one scalar gate logit g_j per raw token and one bias beta_r per offset r in
  the block; block e of m tokens gets weights
  alpha_{e,r} = softmax_r(g_{e*m+r} + beta_r);
* entry = sum_r alpha_{e,r} * x_{e*m+r}, with the same weights for the key,
  the value and the indexer key;
* blocks do not overlap;
* keys are rotated (RoPE) at each raw token's own position before pooling;
  values and indexer keys are not rotated. With m = 1 the pooling is the
  identity, which gives the raw window row.

The entry is rounded to float32 before it is stored or encoded (the precision
in which the encoder takes its decisions).

Parity: pinned in tests by uniform gates giving the block mean, a one-hot gate
giving a single token, invariance to a constant added to all gates or all
biases, m = 1 giving the rotated token, and a pure-Python loop on tiny inputs.

Variants (``compress_variant``): three further readings of the same passages,
each a compressor of its own (the pages cannot decide between them):

* 'overlap' -- [webconsulting], "Kompression und Selektion": CSA groups 4
  tokens and lets information flow across group boundaries. Read as
  overlapping windows: entry e pools the 2m tokens [(e-1)m, (e+1)m), its own
  block and the one before, with one softmax over the 2m gate logits plus a
  learned bias per window offset (2m biases, offsets 0..m-1 the previous
  block). Positions before 0 do not exist: the softmax runs over the tokens
  that do. The entry still ends with its own block, so visibility is unchanged.
* 'rope_after_pool' -- [golem] says only that the last 64 values carry RoPE.
  Read here as pooling the unrotated keys and rotating the pooled key once, at
  the position of the block's last token (e*m + m - 1).
* 'channel_gate' -- [chaosnode]'s softmax gating with a positional bias, read
  per channel: every output channel c (the D key channels, then the D value
  channels, then the indexer-key channels) has its own gate logit per token and
  its own bias per offset, alpha_{e,r,c} = softmax_r(g_{em+r,c} + beta_{r,c}).
  Keys are rotated before pooling, as in the base reading.

Each variant is pinned by a reduction to the base reading (a masked previous
block, m = 1, equal channel gates), closed forms (window means, one-hot
choices, the complex form of the rotation) and a pure-Python loop.
"""

import numpy as np

from . import rope, formats


def gate_weights(gate, pos_bias):
    """gate [..., T] (T % m == 0), pos_bias [m] -> alpha [..., T/m, m] (float64)."""
    pos_bias = np.asarray(pos_bias, np.float32).astype(np.float64)
    m = pos_bias.shape[0]
    g = np.asarray(gate, np.float32).astype(np.float64)
    z = g.reshape(g.shape[:-1] + (g.shape[-1] // m, m)) + pos_bias
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def pool(x, alpha):
    """x [..., T, C], alpha [..., T/m, m] -> [..., T/m, C] weighted sums (float64)."""
    x = np.asarray(x, np.float64)
    n, m = alpha.shape[-2], alpha.shape[-1]
    xr = x.reshape(x.shape[:-2] + (n, m, x.shape[-1]))
    return np.einsum('...em,...emc->...ec', alpha, xr)


def compress(raw_k, raw_v, gate, pos_bias, pos0, base=10000.0, raw_ik=None):
    """Pool a chunk of raw tokens into entries.

    raw_k, raw_v: [B, T, D]; gate: [B, T]; pos_bias: [m]; raw_ik: [B, T, dI] or None.
    pos0 is the position of the first token (pos0 % m == 0, T % m == 0).
    Returns float32 arrays (k [B, T/m, D], v [B, T/m, D], ik [B, T/m, dI] or None);
    entry j of the result is entry number pos0/m + j of the store.
    """
    m = int(np.asarray(pos_bias).shape[0])
    T = np.asarray(raw_k).shape[1]
    assert pos0 % m == 0 and T % m == 0
    pos = pos0 + np.arange(T, dtype=np.int64)
    k_rot = rope.apply(np.asarray(raw_k, np.float64), pos[None, :], base)
    alpha = gate_weights(gate, pos_bias)
    k = pool(k_rot, alpha).astype(np.float32)
    v = pool(raw_v, alpha).astype(np.float32)
    ik = None if raw_ik is None else pool(raw_ik, alpha).astype(np.float32)
    return k, v, ik


def encode_kv(x32, fmt):
    """Encode float32 entries for a store: 'f32' keeps them, 'e4m3_bf16' splits them."""
    if fmt == 'f32':
        return {'f32': np.asarray(x32, np.float32)}
    codes, rope_bits, scale = formats.kv_quantize(x32)
    return {'nope': codes, 'rope': rope_bits, 'scale': scale}


def encode_ik(x32, fmt):
    if fmt == 'f32':
        return {'f32': np.asarray(x32, np.float32)}
    packed, scales = formats.mxfp4_quantize(x32)
    return {'e2m1': packed, 'e8m0': scales}


def decode_kv(store):
    if 'f32' in store:
        return np.asarray(store['f32'], np.float32).astype(np.float64)
    return formats.kv_dequantize(store['nope'], store['rope'], store['scale'])


def decode_ik(store):
    if 'f32' in store:
        return np.asarray(store['f32'], np.float32).astype(np.float64)
    return formats.mxfp4_dequantize(store['e2m1'], store['e8m0'])


VARIANTS = ('block', 'overlap', 'rope_after_pool', 'channel_gate')


def compress_variant(variant, raw_k, raw_v, gate, pos_bias, pos0, base=10000.0, raw_ik=None):
    """A compressor variant over a chunk of whole blocks starting at position pos0.

    'block':            as compress(); gate [B, T], pos_bias [m].
    'overlap':          raw_k, raw_v, raw_ik and gate cover positions [pos0 - m, pos0 + T)
                        (the block before the chunk comes first; ignored when pos0 == 0);
                        pos_bias [2m] over the window offsets.
    'rope_after_pool':  gate [B, T], pos_bias [m]; keys pooled unrotated, then rotated at
                        the block's last position.
    'channel_gate':     gate [B, T, C], pos_bias [m, C], C = D + D (+ dI): the key channels,
                        the value channels, the indexer-key channels.
    Returns float32 (k [B, T/m, D], v [B, T/m, D], ik [B, T/m, dI] or None).
    """
    if variant == 'block':
        return compress(raw_k, raw_v, gate, pos_bias, pos0, base, raw_ik)
    raw_k = np.asarray(raw_k, np.float64)
    raw_v = np.asarray(raw_v, np.float64)
    rik = None if raw_ik is None else np.asarray(raw_ik, np.float64)
    g = np.asarray(gate, np.float32).astype(np.float64)
    bias = np.asarray(pos_bias, np.float32).astype(np.float64)
    B, D = raw_k.shape[0], raw_k.shape[-1]
    if variant == 'overlap':
        m = bias.shape[0] // 2
        T = raw_k.shape[1] - m
        assert pos0 % m == 0 and T % m == 0
        pos = pos0 - m + np.arange(T + m, dtype=np.int64)
        k_rot = rope.apply(raw_k, pos[None, :], base)
        n = T // m
        out_k, out_v = np.empty((B, n, D)), np.empty((B, n, D))
        out_u = None if rik is None else np.empty((B, n, rik.shape[-1]))
        for e in range(n):
            w = slice(e * m, e * m + 2 * m)            # window rows: the block before, then block e
            z = g[:, w] + bias[None, :]
            z = np.where(pos[w][None, :] >= 0, z, -np.inf)   # positions before 0 do not exist
            z = z - z.max(axis=-1, keepdims=True)
            a = np.exp(z)
            a = a / a.sum(axis=-1, keepdims=True)            # [B, 2m]
            out_k[:, e] = np.einsum('br,brc->bc', a, k_rot[:, w])
            out_v[:, e] = np.einsum('br,brc->bc', a, raw_v[:, w])
            if rik is not None:
                out_u[:, e] = np.einsum('br,brc->bc', a, rik[:, w])
        return (out_k.astype(np.float32), out_v.astype(np.float32),
                None if out_u is None else out_u.astype(np.float32))
    if variant == 'rope_after_pool':
        m = bias.shape[0]
        T = raw_k.shape[1]
        assert pos0 % m == 0 and T % m == 0
        alpha = gate_weights(gate, pos_bias)
        k = pool(raw_k, alpha)                                   # unrotated keys pooled
        last = pos0 + m - 1 + m * np.arange(T // m, dtype=np.int64)
        k = rope.apply(k, last[None, :], base)
        v = pool(raw_v, alpha)
        ik = None if rik is None else pool(rik, alpha)
        return k.astype(np.float32), v.astype(np.float32), None if ik is None else ik.astype(np.float32)
    if variant == 'channel_gate':
        m = bias.shape[0]
        T = raw_k.shape[1]
        assert pos0 % m == 0 and T % m == 0
        pos = pos0 + np.arange(T, dtype=np.int64)
        k_rot = rope.apply(raw_k, pos[None, :], base)
        x = np.concatenate([k_rot, raw_v] + ([] if rik is None else [rik]), axis=-1)   # [B, T, C]
        C = x.shape[-1]
        assert g.shape[-1] == C and bias.shape[1] == C
        z = g.reshape(B, T // m, m, C) + bias[None, None]
        z = z - z.max(axis=2, keepdims=True)
        a = np.exp(z)
        a = a / a.sum(axis=2, keepdims=True)                   # softmax over r, per channel
        y = (a * x.reshape(B, T // m, m, C)).sum(axis=2)
        k, v = y[..., :D], y[..., D:2 * D]
        ik = None if rik is None else y[..., 2 * D:]
        return k.astype(np.float32), v.astype(np.float32), None if ik is None else ik.astype(np.float32)
    raise ValueError(f'unknown compressor variant {variant!r}')
