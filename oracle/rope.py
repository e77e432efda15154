"""Rotary position embedding on the last 64 dimensions (oracle side).

[golem], "Komprimierte Erinnerung für längere Kontexte": the last 64 values of
each vector carry RoPE position information (which is why they stay in BF16).
The pages give neither the pair convention nor the base; the reading used is:
dims [D-64, D) rotate in interleaved pairs (D-64+2i, D-64+2i+1), i < 32, by
angle p * base^(-2i/64), base 10000 (the value the small fp32 configuration
names). Angles are formed in float64 because p * theta reaches 1e6 radians at
a million positions, beyond what float32 resolves.

Parity: pinned in tests by norm preservation of every pair, dependence of
<R(p)q, R(p')k> on p - p' only, the identity at p = 0, and agreement with
multiplication by exp(i*angle) in complex arithmetic.
"""

import numpy as np

from .formats import ROPE_DIM


def inv_freq(base=10000.0, rope_dim=ROPE_DIM):
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / rope_dim)


def apply(x, pos, base=10000.0):
    """Rotate the last 64 dims of x [..., D] at positions pos (broadcast to x[..., 0])."""
    x = np.asarray(x, np.float64)
    pos = np.asarray(pos, np.float64)
    ang = pos[..., None] * inv_freq(base)[(None,) * pos.ndim]
    c, s = np.cos(ang), np.sin(ang)
    out = x.copy()
    d0 = x.shape[-1] - ROPE_DIM
    xe = x[..., d0 + 0::2]
    xo = x[..., d0 + 1::2]
    out[..., d0 + 0::2] = xe * c - xo * s
    out[..., d0 + 1::2] = xe * s + xo * c
    return out
