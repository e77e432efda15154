"""Pins of the oracle's number formats against independent references.

References: torch's float8_e4m3fn and bfloat16 conversions (library routines),
brute-force nearest-value search over every code, and the OCP landmark values
in tests/golden/ocp_landmarks.txt.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), 'golden')


def _landmarks():
    rows = []
    for line in open(os.path.join(GOLDEN, 'ocp_landmarks.txt')):
        line = line.split('#')[0].strip()
        if line:
            fmt, code, val = line.split()
            rows.append((fmt, int(code, 16), float(val)))
    return rows


@pytest.mark.parametrize('fmt,code,val', _landmarks())
def test_ocp_landmarks(fmt, code, val):
    dec = {'e4m3': F.e4m3_decode, 'e2m1': F.e2m1_decode, 'e8m0': F.e8m0_decode}[fmt]
    got = float(np.asarray(dec(np.array([code])))[0])
    if math.isnan(val):
        assert math.isnan(got)
    else:
        assert got == val and math.copysign(1, got) == math.copysign(1, val)


def test_e4m3_decode_matches_torch_all_codes():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = F.e4m3_decode(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_e4m3_encode_matches_torch_in_range():
    g = np.random.default_rng(5)
    x = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(30),
        g.standard_normal(50000).astype(np.float32) * np.float32(0.01),     # subnormal range
        (F.E4M3_VALUES[:126] + F.E4M3_VALUES[1:127]).astype(np.float32) / 2,  # exact midpoints
        -(F.E4M3_VALUES[:126] + F.E4M3_VALUES[1:127]).astype(np.float32) / 2,
        np.array([0.0, -0.0, 447.99, 463.99, -463.99], np.float32),
    ]).astype(np.float32)
    x = x[np.abs(x) < 464]          # torch rounds (448, 464) to 448; beyond it gives NaN
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(F.e4m3_encode(x), ref)


def test_e4m3_encode_brute_force_and_saturation():
    g = np.random.default_rng(6)
    x = (g.standard_normal(3000) * 100).astype(np.float32)
    x = np.concatenate([x, np.array([448.0, 500.0, 1e30, np.inf, -np.inf, -1e9], np.float32)])
    got = F.e4m3_encode(x)
    finite_codes = [c for c in range(256) if not np.isnan(F.E4M3_VALUES[c])]
    for xi, ci in zip(x.astype(np.float64), got):
        a = min(abs(xi), 448.0)
        best = None
        for c in finite_codes:
            v = F.E4M3_VALUES[c]
            if np.signbit(v) != np.signbit(xi):
                continue
            d = abs(abs(v) - a)
            key = (d, c & 1)                      # ties go to the even code
            if best is None or key < best[0]:
                best = (key, c)
        assert ci == best[1], (xi, ci, best)
    assert F.e4m3_encode(np.array([np.nan], np.float32))[0] == 0x7F


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes).astype(np.float32)), codes)


def test_bf16_encode_matches_torch():
    g = np.random.default_rng(7)
    x = np.concatenate([
        g.standard_normal(100000).astype(np.float32),
        (g.standard_normal(1000) * 1e-39).astype(np.float32),
        np.array([np.inf, -np.inf, 3.4028235e38, 0.0, -0.0, 1.0000001, 1.00390625, 1.01171875], np.float32),
    ])
    # exact midpoints between consecutive bf16 values
    u = (g.integers(0, 0x7F7F, 5000).astype(np.uint32) << 16) | 0x8000
    x = np.concatenate([x, u.view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.bf16_encode(x), ref)
    nan = F.bf16_encode(np.array([np.nan], np.float32))
    assert np.isnan(F.bf16_decode(nan))[0]


def test_e2m1_encode_brute_force():
    g = np.random.default_rng(8)
    v = np.concatenate([g.uniform(-8, 8, 20000),
                        np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0, 6.0, 7.9, -7.0])])
    got = F.e2m1_encode(v)
    for vi, ci in zip(v, got):
        a = min(abs(vi), 6.0)
        cands = [(abs(F.E2M1_VALUES[c] - a), c & 1, c) for c in range(8)]
        best = min(cands)[2] | (8 if vi < 0 else 0)
        assert ci == best, (vi, ci, best)


def test_mx_scale_rule():
    g = np.random.default_rng(9)
    x = (g.standard_normal((400, 64)) * np.exp(g.uniform(-20, 20, (400, 1)))).astype(np.float32)
    x[0] = 0.0
    x[1, :32] = 0.0
    packed, scales = F.mxfp4_quantize(x)
    deq = F.mxfp4_dequantize(packed, scales)
    blocks = x.reshape(400, 2, 32).astype(np.float64)
    for r in range(400):
        for b in range(2):
            amax = np.abs(blocks[r, b]).max()
            e = -127 if amax == 0 else max(-127, math.frexp(float(amax))[1] - 1 - 2)
            assert scales[r, b] == e + 127
            step = 2.0 ** e
            err = np.abs(deq[r, 32 * b:32 * b + 32] - blocks[r, b])
            # values up to 6*2^E round within half of the largest quantum (2*2^E);
            # values in (6, 8)*2^E are clipped to 6*2^E.
            assert np.all(err <= np.maximum(1.0 * step, np.abs(blocks[r, b]) - 6 * step) + 1e-300)
            if amax > 0:
                assert np.abs(deq[r, 32 * b:32 * b + 32]).max() >= 4 * step


def test_mxfp4_nibble_order():
    x = np.zeros((1, 32), np.float32)
    x[0, 0] = 1.0     # code 2 -> low nibble of byte 0
    x[0, 1] = 6.0     # code 7 -> high nibble of byte 0
    x[0, 2] = -0.5    # code 9 -> low nibble of byte 1
    packed, scales = F.mxfp4_quantize(x)
    assert scales[0, 0] == 127 and packed[0, 0] == 0x72 and packed[0, 1] & 0xF == 0x9


def test_fp8_row_quantize_error_bound():
    g = np.random.default_rng(10)
    x = (g.standard_normal((300, 192)) * np.exp(g.uniform(-5, 5, (300, 1)))).astype(np.float32)
    x[3] = 0.0
    codes, rope_bits, s = F.kv_quantize(x)
    assert codes.shape == (300, 128) and rope_bits.shape == (300, 64) and s.shape == (300, 1)
    deq = F.kv_dequantize(codes, rope_bits, s)
    nope = x[:, :128].astype(np.float64)
    amax = np.abs(nope).max(1)
    assert s[3, 0] == 1.0
    # normal E4M3 range: relative error <= 2^-4; subnormal range: half the quantum 2^-9 * s
    err = np.abs(deq[:, :128] - nope)
    bound = np.maximum(2.0 ** -4 * np.abs(nope), 2.0 ** -10 * s.astype(np.float64)) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the largest element of each row maps to the largest code
    big = np.argmax(np.abs(nope), 1)
    assert np.all((codes[np.arange(300), big] & 0x7F)[amax > 0] == 0x7E)
    assert np.array_equal(deq[:, 128:], torch.from_numpy(x[:, 128:]).to(torch.bfloat16).double().numpy())


def test_fp8_row_scale_nan_group_propagates():
    """A NaN anywhere in a 128-dim group makes the group's scale NaN and every code of the
    group the E4M3 NaN code 0x7F (x / NaN is NaN); another group and the BF16 RoPE dims
    are unaffected. An infinite element makes the scale infinite: its own code is NaN
    (inf / inf) and every finite element of the group becomes a zero code."""
    x = np.zeros((3, 192), np.float32)
    x[:, :128] = np.linspace(-2, 2, 128, dtype=np.float32)
    x[:, 128:] = 0.75
    x[1, 17] = np.nan
    x[2, 5] = np.inf
    assert np.isnan(F.fp8_row_scale(np.array([np.nan], np.float32)))[0]
    assert F.fp8_row_scale(np.array([0.0], np.float32))[0] == 1.0
    assert F.fp8_row_scale(np.array([448.0], np.float32))[0] == 1.0
    codes, rope_bits, s = F.kv_quantize(x)
    assert s[0, 0] == np.float32(2.0) / np.float32(448.0)
    assert np.isnan(s[1, 0]) and np.all(codes[1] == 0x7F)
    assert np.isinf(s[2, 0]) and codes[2, 5] == 0x7F
    assert np.all((codes[2, np.arange(128) != 5] & 0x7F) == 0)
    assert np.array_equal(codes[0], F.e4m3_encode(x[0, :128] / s[0, 0]))
    assert np.all(F.bf16_decode(rope_bits) == 0.75)
