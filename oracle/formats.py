"""Number formats of the compressed caches: E4M3, BF16, E2M1, E8M0 (oracle side).

[chaosnode], section "Hybrid Attention: CSA und HCA": cache entries are held
mostly in FP8, the RoPE dimensions in BF16, and the indexer runs in FP4.
[golem], "Komprimierte Erinnerung für längere Kontexte": the last 64 values of
a vector carry RoPE and are kept in BF16; the introduction names MXFP4 for the
attention mechanism.

The pages do not define the formats; the definitions are the OCP ones:

* E4M3 (OFP8 rev 1.0, "E4M3"): bias 7, three mantissa bits, no infinities,
  S.1111.111 is NaN, largest finite 448, subnormals m/8 * 2^-6. Encoding
  rounds to nearest, ties to even, and saturates finite overflow to +-448
  (the spec's saturating mode). NaN encodes as 0x7F.
* BF16: the top 16 bits of a float32 after round-to-nearest-even.
* E2M1 (MX v1.0 element format): magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6};
  round to nearest even, saturate to +-6.
* E8M0 (MX v1.0 scale format): 2^(c-127); 0xFF is NaN.
* MX block scale (MX v1.0 section 6.3): for a block of 32 values with largest
  magnitude amax, shared exponent E = floor(log2(amax)) - 2 (2 is the largest
  exponent of E2M1), clamped to [-127, 127]; amax == 0 gives E = -127. Each
  element is x / 2^E encoded as E2M1. A block holding NaN or Inf gets scale
  0xFF and zero elements.

The FP8 row scale is a reading (the configuration asks for "a per-128 scale"
without a format): s = amax / 448 in float32 (amax == 0 gives s = 1, a NaN in
the group gives s = NaN), codes are E4M3(x / s) with IEEE float32 division.

Parity: every codec is pinned in the test suite against torch's float8_e4m3fn
and bfloat16 conversions, brute-force nearest-value search, and the OCP
landmark values in tests/golden/.
"""

import numpy as np

ROPE_DIM = 64          # [golem]: the last 64 values carry RoPE, kept in BF16
FP8_GROUP = 128        # per-128 FP8 scale group (configuration text)
MX_BLOCK = 32          # MX v1.0 block size
E4M3_MAX = 448.0
E2M1_MAX = 6.0


# ----------------------------------------------------------------- E4M3 ----

def _e4m3_table():
    """Value of every E4M3 code (NaN for S.1111.111)."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
_E4M3_POS = E4M3_VALUES[:127]          # codes 0..126, ascending magnitudes


def e4m3_decode(codes):
    return E4M3_VALUES[np.asarray(codes, np.uint8)]


def e4m3_encode(x):
    """float32 array -> E4M3 codes, round-to-nearest-even, saturating."""
    x = np.asarray(x, np.float32).astype(np.float64)
    nan = np.isnan(x)
    neg = np.signbit(x)
    a = np.abs(np.where(nan, 0.0, x))
    a = np.minimum(a, E4M3_MAX * 2)       # keep Inf finite; saturated below
    _, ex = np.frexp(np.maximum(a, 2.0 ** -6))
    quantum = np.ldexp(1.0, (ex - 1) - 3)  # 3 mantissa bits; subnormal quantum 2^-9
    r = np.rint(a / quantum) * quantum     # exact: division by a power of two
    r = np.minimum(r, E4M3_MAX)
    code = np.searchsorted(_E4M3_POS, r).astype(np.uint8)
    code = np.where(neg, code | 0x80, code).astype(np.uint8)
    return np.where(nan, np.uint8(0x7F), code).astype(np.uint8)


# ----------------------------------------------------------------- BF16 ----

def bf16_encode(x):
    """float32 array -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(np.asarray(x, np.float32)).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(nan, (u >> 16) | 0x40, r)
    return (r & 0xFFFF).astype(np.uint16)


def bf16_decode(h):
    h = np.asarray(h, np.uint16).astype(np.uint32) << 16
    return h.view(np.float32).astype(np.float64)


def bf16_round(x):
    """float32 -> nearest bfloat16 value, as float64."""
    return bf16_decode(bf16_encode(x))


# ------------------------------------------------------------ E2M1/E8M0 ----

E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                        -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def e2m1_decode(codes):
    return E2M1_VALUES[np.asarray(codes, np.uint8) & 0xF]


def e2m1_encode(v):
    """float array (already divided by the block scale) -> E2M1 codes (0..15)."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    quantum = np.where(a < 2.0, 0.5, np.where(a < 4.0, 1.0, 2.0))
    r = np.minimum(np.rint(a / quantum) * quantum, E2M1_MAX)
    mag = np.searchsorted(E2M1_VALUES[:8], r).astype(np.uint8)
    return np.where(np.signbit(v), mag | 8, mag).astype(np.uint8)


def e8m0_decode(c):
    c = np.asarray(c, np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mx_scale_exponent(amax):
    """Shared exponent of an MXFP4 block from its float32 amax (MX v1.0 6.3)."""
    amax = np.asarray(amax, np.float32).astype(np.float64)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    e = np.where(amax > 0, (ex - 1) - 2, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def mxfp4_quantize(x):
    """float32 [..., d] (d % 32 == 0) -> (packed E2M1 bytes [..., d/2], E8M0 [..., d/32]).

    Byte i of a row holds element 2i in its low nibble and 2i+1 in its high nibble.
    """
    x = np.asarray(x, np.float32)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)).astype(np.float64)
    bad = ~np.isfinite(blocks).all(axis=-1)
    amax = np.abs(np.where(np.isfinite(blocks), blocks, 0.0)).max(axis=-1)
    e = mx_scale_exponent(amax)
    codes = e2m1_encode(blocks / np.ldexp(1.0, e)[..., None])
    codes = np.where(bad[..., None], np.uint8(0), codes)
    scales = np.where(bad, 255, e + 127).astype(np.uint8)
    codes = codes.reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scales


def mxfp4_unpack(packed):
    packed = np.asarray(packed, np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def mxfp4_dequantize(packed, scales):
    vals = e2m1_decode(mxfp4_unpack(packed))
    d = vals.shape[-1]
    s = e8m0_decode(scales)
    vals = vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)) * s[..., None]
    return vals.reshape(vals.shape[:-2] + (d,))


# ------------------------------------------------ FP8 + BF16 KV split -------

def fp8_row_scale(amax):
    """amax / 448 in float32; 1 for an all-zero group; NaN when the group holds a NaN."""
    amax = np.asarray(amax, np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax > 0, s, np.float32(1.0))
    return np.where(np.isnan(amax), np.float32(np.nan), s).astype(np.float32)


def kv_quantize(x):
    """float32 [..., D] -> (e4m3 codes [..., D-64], bf16 bits [..., 64], scales [..., (D-64)/128]).

    Dims [0, D-64) are stored as E4M3 with one float32 scale per 128 dims;
    the last 64 dims (the RoPE dims) are stored as BF16.
    """
    x = np.asarray(x, np.float32)
    dn = x.shape[-1] - ROPE_DIM
    assert dn > 0 and dn % FP8_GROUP == 0
    nope = x[..., :dn].reshape(x.shape[:-1] + (dn // FP8_GROUP, FP8_GROUP))
    amax = np.abs(nope).max(axis=-1)
    s = fp8_row_scale(amax)
    q = (nope / s[..., None]).astype(np.float32)       # IEEE float32 division
    codes = e4m3_encode(q).reshape(x.shape[:-1] + (dn,))
    return codes, bf16_encode(x[..., dn:]), s


def kv_dequantize(codes, rope_bits, scales):
    codes = np.asarray(codes, np.uint8)
    dn = codes.shape[-1]
    v = e4m3_decode(codes).reshape(codes.shape[:-1] + (dn // FP8_GROUP, FP8_GROUP))
    v = v * np.asarray(scales, np.float32).astype(np.float64)[..., None]
    return np.concatenate([v.reshape(codes.shape[:-1] + (dn,)), bf16_decode(rope_bits)], axis=-1)
