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
