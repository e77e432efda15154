"""Pins of the oracle's compression, scoring, selection and attention.

Each check compares the oracle with something other than itself: a closed form
(block mean, one-hot gate, the hand-derived example in
tests/golden/pool_worked_example.txt), an invariant (RoPE norms and relative
positions, softmax shift invariance), a pure-Python loop on tiny inputs, exact
rational arithmetic (MXFP4 dot products), or torch's scaled-dot-product
attention in float64 (dense causal, sliding-window and duplicated-key forms).
"""

import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import compress as C
from oracle import formats as F
from oracle import indexer as I
from oracle import model as M
from oracle import rope as R

GOLDEN = os.path.join(os.path.dirname(__file__), 'golden')


# ------------------------------------------------------------------ RoPE ----

def test_rope_identity_at_zero_and_norms():
    g = np.random.default_rng(0)
    x = g.standard_normal((5, 192))
    assert np.array_equal(R.apply(x, np.zeros(5, np.int64)), x)
    y = R.apply(x, np.array([1, 7, 4095, 65535, 1048575]))
    assert np.array_equal(y[:, :128], x[:, :128])
    pn = lambda z: z[:, 128::2] ** 2 + z[:, 129::2] ** 2
    assert np.allclose(pn(y), pn(x), rtol=1e-13, atol=0)


def test_rope_relative_position():
    g = np.random.default_rng(1)
    q, k = g.standard_normal(128), g.standard_normal(128)
    ref = R.apply(q, np.int64(1000)) @ R.apply(k, np.int64(990))
    for p in (10, 5000, 1048575):
        assert abs(R.apply(q, np.int64(p)) @ R.apply(k, np.int64(p - 10)) - ref) < 1e-9


def test_rope_complex_multiplication():
    g = np.random.default_rng(2)
    x = g.standard_normal((3, 128))
    pos = np.array([3, 100000, 1048575])
    y = R.apply(x, pos, 10000.0)
    z = x[:, 64::2] + 1j * x[:, 65::2]
    theta = np.array([10000.0 ** (-(2 * i) / 64) for i in range(32)])
    zz = z * np.exp(1j * (pos[:, None] * theta[None, :]))
    assert np.allclose(y[:, 64::2], zz.real, atol=1e-12) and np.allclose(y[:, 65::2], zz.imag, atol=1e-12)


# --------------------------------------------------------------- pooling ----

def test_pool_worked_example():
    x = np.array([[[1.0], [2.0], [3.0], [4.0]]])
    l5 = math.log(5.0)
    a1 = C.gate_weights(np.array([[0, 0, 0, l5]], np.float32), np.zeros(4, np.float32))
    a2 = C.gate_weights(np.array([[0, 0, 0, l5]], np.float32), np.array([l5, 0, 0, -l5], np.float32))
    assert abs(C.pool(x, a1)[0, 0, 0] - 3.25) < 1e-6
    assert abs(C.pool(x, a2)[0, 0, 0] - 1.75) < 1e-6
    lines = [l for l in open(os.path.join(GOLDEN, 'pool_worked_example.txt')) if l.startswith('case')]
    assert [float(l.split()[-1]) for l in lines] == [3.25, 1.75]


@pytest.mark.parametrize('m', [1, 2, 4, 8, 128])
def test_pool_uniform_gate_is_block_mean(m):
    g = np.random.default_rng(m)
    T = 4 * m
    k = g.standard_normal((2, T, 192)).astype(np.float32)
    v = g.standard_normal((2, T, 192)).astype(np.float32)
    gate = np.full((2, T), 0.7, np.float32)
    beta = np.full(m, -0.3, np.float32)
    ek, ev, _ = C.compress(k, v, gate, beta, pos0=8 * m)
    mean_v = v.reshape(2, 4, m, 192).mean(2)
    assert np.allclose(ev, mean_v, rtol=1e-6, atol=1e-6)
    rot = R.apply(k.astype(np.float64), (8 * m + np.arange(T))[None, :])
    assert np.allclose(ek, rot.reshape(2, 4, m, 192).mean(2), rtol=1e-6, atol=1e-6)


def test_pool_one_hot_and_shift_invariance():
    g = np.random.default_rng(3)
    v = g.standard_normal((1, 8, 128)).astype(np.float32)
    gate = np.zeros((1, 8), np.float32)
    gate[0, 2] = 200.0
    gate[0, 7] = 200.0
    _, ev, _ = C.compress(v, v, gate, np.zeros(4, np.float32), 0)
    assert np.allclose(ev[0, 0], v[0, 2]) and np.allclose(ev[0, 1], v[0, 7])
    # dyadic values, so that the shifted inputs are exact in float32
    gate = (np.round(g.standard_normal((1, 8)) * 1024) / 1024).astype(np.float32)
    beta = (np.round(g.standard_normal(4) * 1024) / 1024).astype(np.float32)
    a = C.gate_weights(gate, beta)
    b = C.gate_weights(gate + np.float32(3.0), beta - np.float32(1.5))
    assert np.allclose(a, b, rtol=1e-12, atol=0)


def test_pool_m1_is_rotated_token():
    g = np.random.default_rng(4)
    k = g.standard_normal((1, 5, 128)).astype(np.float32)
    ek, ev, _ = C.compress(k, k, g.standard_normal((1, 5)).astype(np.float32), np.array([0.3], np.float32), 17)
    assert np.array_equal(ev, k)
    assert np.array_equal(ek, R.apply(k.astype(np.float64), (17 + np.arange(5))[None, :]).astype(np.float32))


def test_pool_python_loop():
    g = np.random.default_rng(5)
    m, T, D = 4, 8, 128
    k = g.standard_normal((1, T, D)).astype(np.float32)
    v = g.standard_normal((1, T, D)).astype(np.float32)
    u = g.standard_normal((1, T, 64)).astype(np.float32)
    gate = g.standard_normal((1, T)).astype(np.float32)
    beta = (0.1 * g.standard_normal(m)).astype(np.float32)
    ek, ev, eu = C.compress(k, v, gate, beta, pos0=400, raw_ik=u)
    for e in range(T // m):
        z = [float(gate[0, e * m + r]) + float(beta[r]) for r in range(m)]
        mx = max(z)
        ex = [math.exp(zz - mx) for zz in z]
        alpha = [x / sum(ex) for x in ex]
        for d in range(D):
            acc_v = sum(alpha[r] * float(v[0, e * m + r, d]) for r in range(m))
            assert abs(acc_v - ev[0, e, d]) <= 1e-6 * max(1, abs(acc_v))
        for i in range(32):
            acc_x = acc_y = 0.0
            for r in range(m):
                p = 400 + e * m + r
                ang = p * 10000.0 ** (-2 * i / 64)
                x0, y0 = float(k[0, e * m + r, 64 + 2 * i]), float(k[0, e * m + r, 65 + 2 * i])
                acc_x += alpha[r] * (x0 * math.cos(ang) - y0 * math.sin(ang))
                acc_y += alpha[r] * (x0 * math.sin(ang) + y0 * math.cos(ang))
            assert abs(acc_x - ek[0, e, 64 + 2 * i]) <= 1e-6 and abs(acc_y - ek[0, e, 65 + 2 * i]) <= 1e-6
        for d in range(64):
            acc_u = sum(alpha[r] * float(u[0, e * m + r, d]) for r in range(m))
            assert abs(acc_u - eu[0, e, d]) <= 1e-6 * max(1, abs(acc_u))


# --------------------------------------------------------------- indexer ----

def test_index_scores_python_loop():
    g = np.random.default_rng(6)
    H, d, N = 3, 8, 11
    iq, w, keys = g.standard_normal((H, d)), g.uniform(-1, 1, H).astype(np.float32), g.standard_normal((N, d))
    got = I.index_scores(iq, w, keys)
    for e in range(N):
        ref = 0.0
        for h in range(H):
            dot = sum(iq[h, j] * keys[e, j] for j in range(d))
            ref += float(w[h]) * (dot if dot > 0 else 0.0)
        assert abs(ref - got[e]) < 1e-12


def test_mxfp4_dot_products_are_exact():
    g = np.random.default_rng(7)
    x = (g.standard_normal((6, 128)) * 3).astype(np.float32)
    y = (g.standard_normal((9, 128)) * 0.01).astype(np.float32)
    px, sx = F.mxfp4_quantize(x)
    py, sy = F.mxfp4_quantize(y)
    dx, dy = F.mxfp4_dequantize(px, sx), F.mxfp4_dequantize(py, sy)
    cx, cy = F.mxfp4_unpack(px), F.mxfp4_unpack(py)
    got = dx @ dy.T
    half = {c: Fraction(int(round(2 * abs(F.E2M1_VALUES[c])))) * (-1 if c & 8 else 1) for c in range(16)}
    for i in range(6):
        for j in range(9):
            tot = Fraction(0)
            for b in range(4):
                e = int(sx[i, b]) - 127 + int(sy[j, b]) - 127
                s = sum(half[cx[i, 32 * b + t]] * half[cy[j, 32 * b + t]] for t in range(32))
                tot += s * (Fraction(2) ** e) / 4     # each element is (half-units)/2
            assert Fraction(got[i, j]) == tot


def test_topk_brute_force_and_ties():
    g = np.random.default_rng(8)
    for trial in range(50):
        n = int(g.integers(1, 300))
        k = int(g.integers(1, 80))
        s = np.round(g.standard_normal(n + 5) * 4) / 4          # many exact ties
        if trial % 7 == 0:
            s[:n // 2] = 0.0
            s[1] = -0.0
        sel = I.topk_select(s, n, k)
        order = sorted(range(n), key=lambda e: (-float(np.float32(s[e])), e))[:min(k, n)]
        ref = np.full(k, -1, np.int32)
        ref[:len(order)] = sorted(order)
        assert np.array_equal(sel, ref)


def test_topk_nan_ranks_last():
    s = np.array([1.0, np.nan, 0.5, -np.inf, 2.0])
    assert list(I.topk_select(s, 5, 4)) == [0, 2, 3, 4]


def _mx_keys_with_dots(dots_h0, dots_h1):
    """Queries and MXFP4 keys (32 dims, one block each) whose dot products with the two
    query heads are the given small integers: head 0 reads dim 0, head 1 reads dim 1."""
    n = len(dots_h0)
    iq = np.zeros((2, 32), np.float32)
    iq[0, 0] = 1.0
    iq[1, 1] = 1.0
    keys = np.zeros((n, 32), np.float32)
    keys[:, 0] = dots_h0
    keys[:, 1] = dots_h1
    keys[:, 2] = 4.0                      # keeps every block's scale at 2^0 (amax 4 -> E = 0)
    return iq, keys


def test_index_scores_nan_key_block_propagates():
    """A key whose MXFP4 block scale is NaN (E8M0 0xFF) decodes to NaN, so every dot
    product with it is NaN and, with max(0, x) propagating NaN, so is its score: it
    ranks below every number. Hand-derived: w = (1, 1), dots (h0, h1) per key
    0: (3, 0), 1: (1, 1), 2: (0, 6) with a NaN block, 3: (2, 2), 4: (-1, 0), 5: (0, 2).
    Scores 3, 2, NaN, 4, 0, 2 -> top-3 = {0, 3} plus the lower of the tied 1 and 5 = {0, 1, 3}.
    Under the other reading (a NaN dot product counted as 0) key 2 would score 6 and be
    selected instead of key 1."""
    iq, keys = _mx_keys_with_dots([3, 1, 0, 2, -1, 0], [0, 1, 6, 2, 0, 2])
    packed, sc = F.mxfp4_quantize(keys)
    assert np.all(sc == 127)
    sc = sc.copy()
    sc[2, 0] = 0xFF
    dk = F.mxfp4_dequantize(packed, sc)
    assert np.isnan(dk[2]).all() and np.isfinite(np.delete(dk, 2, 0)).all()
    ip, isc = F.mxfp4_quantize(iq)
    s = I.index_scores(F.mxfp4_dequantize(ip, isc), np.ones(2, np.float32), dk)
    assert np.isnan(s[2]) and list(s[[0, 1, 3, 4, 5]]) == [3.0, 2.0, 4.0, 0.0, 2.0]
    assert list(I.topk_select(s, 6, 3)) == [0, 1, 3]
    assert list(I.topk_select(s, 6, 6)) == [0, 1, 2, 3, 4, 5]
    assert I.kth_score(s, 6, 3) == 2.0 and I.kth_score(s, 6, 6) == -np.inf


def test_index_scores_nan_query_head_propagates():
    """A NaN block in one query head makes that head's dot product NaN for every key,
    so every score is NaN (even where the head's weight is 0: 0 * NaN = NaN) and the
    selection is the k lowest ids. Hand-derived, same keys as above: top-3 = {0, 1, 2}."""
    iq, keys = _mx_keys_with_dots([3, 1, 0, 2, -1, 0], [0, 1, 6, 2, 0, 2])
    packed, sc = F.mxfp4_quantize(keys)
    ip, isc = F.mxfp4_quantize(iq)
    isc = isc.copy()
    isc[1, 0] = 0xFF
    for w in (np.ones(2, np.float32), np.array([1.0, 0.0], np.float32)):
        s = I.index_scores(F.mxfp4_dequantize(ip, isc), w, F.mxfp4_dequantize(packed, sc))
        assert np.isnan(s).all()
        assert list(I.topk_select(s, 6, 3)) == [0, 1, 2]
        assert I.kth_score(s, 6, 3) == -np.inf


def test_index_scores_negative_and_zero_dots():
    """max(0, x) clamps negative dot products and -0 to +0 (no NaN involved): one head
    with dots -5, -0.0, 7 and weight 2 gives scores 0, 0, 14."""
    iq = np.array([[1.0, 0.0]])
    keys = np.array([[-5.0, 1.0], [-0.0, 3.0], [7.0, -2.0]])
    s = I.index_scores(iq, np.array([2.0], np.float32), keys)
    assert list(s) == [0.0, 0.0, 14.0] and not np.signbit(s[1])


def _kth_brute(scores, n_vis, k):
    """k-th score by a plain sort of (rank class, value, id), NaN in the lowest class."""
    vals = [float(np.float32(x)) for x in scores[:n_vis]]
    order = sorted(range(n_vis), key=lambda e: (math.isnan(vals[e]), -(0.0 if math.isnan(vals[e]) else vals[e]), e))
    v = vals[order[min(k, n_vis) - 1]]
    return -math.inf if math.isnan(v) else v


def test_kth_score_brute_force_ties_zero_nan():
    g = np.random.default_rng(31)
    for trial in range(200):
        n = int(g.integers(1, 60))
        k = int(g.integers(1, 70))
        s = np.round(g.standard_normal(n + 3) * 2) / 2          # many exact ties
        s[g.random(n + 3) < 0.15] = np.nan
        s[g.random(n + 3) < 0.1] = -0.0
        s[g.random(n + 3) < 0.1] = 0.0
        if trial % 5 == 0:
            s[:n] = np.nan
        got, ref = I.kth_score(s, n, k), _kth_brute(s, n, k)
        assert got == ref, (trial, got, ref)
        # every selected id scores at or above the k-th score, every other visible one at or below
        sel = I.topk_select(s, n, k)
        sel = sel[sel >= 0]
        key = lambda e: -math.inf if math.isnan(s[e]) else float(np.float32(s[e]))
        assert all(key(e) >= got for e in sel)
        assert all(key(e) <= got for e in set(range(n)) - set(sel.tolist()))
    # hand-checked: ties straddling the boundary, -0 equal to +0, scores rounded to float32
    assert I.kth_score(np.array([1.0, 2.0, 2.0, 2.0, 0.5]), 5, 2) == 2.0
    assert I.kth_score(np.array([-0.0, 0.0, -1.0]), 3, 2) == 0.0
    assert I.kth_score(np.array([1.0 + 1e-12, 1.0, 3.0]), 3, 3) == 1.0
    assert I.kth_score(np.array([np.nan, 5.0, np.nan]), 3, 1) == 5.0
    assert I.kth_score(np.array([np.nan, 5.0, np.nan]), 3, 2) == -np.inf
    assert I.kth_score(np.array([4.0, 9.0]), 1, 5) == 4.0          # fewer visible than k


# ------------------------------------------------------------- attention ----

def _sdpa(q, K, V, scale, mask=None):
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(K)[None], torch.from_numpy(V)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask)[None], scale=scale)
    return out[0].numpy()


def _raw_case(seed, T, D=128, H=4):
    g = np.random.default_rng(seed)
    k = (g.standard_normal((1, T, D)) / 8).astype(np.float32)
    v = g.standard_normal((1, T, D)).astype(np.float32)
    q = (g.standard_normal((H, D)) / 8).astype(np.float32)
    return k, v, q


@pytest.mark.parametrize('T,t', [(40, 39), (40, 17), (9, 0)])
def test_m1_all_selected_no_window_is_dense_causal(T, t):
    k, v, q = _raw_case(T + t, T)
    caches = M.build_caches(k, v, np.zeros((1, T), np.float32), np.zeros(1, np.float32), 'f32')
    o, lse = A.attend_query(q, t, np.arange(t + 1), caches['dk'][0], caches['dv'][0],
                            caches['dwk'][0], caches['dwv'][0], W=0)
    qr = R.apply(q.astype(np.float64), np.int64(t))
    kr = R.apply(k[0].astype(np.float64), np.arange(T))[:t + 1]
    ref = _sdpa(qr, kr, v[0, :t + 1].astype(np.float64), 1 / math.sqrt(128))
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize('W', [1, 5, 128])
def test_m1_all_selected_with_window_duplicates_keys(W):
    T, t = 60, 50
    k, v, q = _raw_case(W, T)
    caches = M.build_caches(k, v, np.zeros((1, T), np.float32), np.zeros(1, np.float32), 'f32')
    o, _ = A.attend_query(q, t, np.arange(t + 1), caches['dk'][0], caches['dv'][0],
                          caches['dwk'][0], caches['dwv'][0], W=W)
    qr = R.apply(q.astype(np.float64), np.int64(t))
    kr = R.apply(k[0].astype(np.float64), np.arange(T))[:t + 1]
    mask = np.zeros((q.shape[0], t + 1))
    mask[:, max(0, t - W + 1):] = math.log(2.0)   # a key present twice weighs twice
    ref = _sdpa(qr, kr, v[0, :t + 1].astype(np.float64), 1 / math.sqrt(128), mask)
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6)


def test_window_only_is_sliding_window_attention():
    T, t, W = 300, 250, 128
    k, v, q = _raw_case(11, T)
    caches = M.build_caches(k, v, g := np.random.default_rng(1).standard_normal((1, T)).astype(np.float32),
                            np.zeros(4, np.float32), 'f32')
    o, _ = M.window_query(q, t, caches['dwk'][0], caches['dwv'][0], W)
    o2, _ = M.hca_query(q, t, caches['dk'][0], caches['dv'][0], caches['dwk'][0], caches['dwv'][0], 4, W,
                        n_entries=0)
    qr = R.apply(q.astype(np.float64), np.int64(t))
    kr = R.apply(k[0].astype(np.float64), np.arange(T))[t - W + 1:t + 1]
    ref = _sdpa(qr, kr, v[0, t - W + 1:t + 1].astype(np.float64), 1 / math.sqrt(128))
    assert np.allclose(o, ref, rtol=1e-6, atol=1e-6) and np.array_equal(o, o2)
    # before the first block completes a CSA/HCA layer is window-only as well
    o3, _ = M.hca_query(q, 2, caches['dk'][0], caches['dv'][0], caches['dwk'][0], caches['dwv'][0], 4, W)
    o4, _ = M.window_query(q, 2, caches['dwk'][0], caches['dwv'][0], W)
    assert np.array_equal(o3, o4)


def test_single_key_returns_its_value():
    g = np.random.default_rng(12)
    V = g.standard_normal((1, 192))
    o, lse = A.attend(g.standard_normal((7, 192)), g.standard_normal((1, 192)), V, 0.1)
    assert np.allclose(o, np.repeat(V, 7, 0), rtol=1e-15, atol=0)


def test_csa_with_all_selected_equals_hca():
    g = np.random.default_rng(13)
    T, m, t = 256, 4, 255
    k = g.standard_normal((1, T, 192)).astype(np.float32)
    v = g.standard_normal((1, T, 192)).astype(np.float32)
    u = g.standard_normal((1, T, 128)).astype(np.float32)
    caches = M.build_caches(k, v, g.standard_normal((1, T)).astype(np.float32),
                            (0.1 * g.standard_normal(m)).astype(np.float32), 'e4m3_bf16', raw_ik=u, ik_fmt='mxfp4')
    q = g.standard_normal((8, 192)).astype(np.float32)
    iq = F.mxfp4_dequantize(*F.mxfp4_quantize(g.standard_normal((4, 128)).astype(np.float32)))
    w = g.uniform(0, 1, 4).astype(np.float32)
    o1, l1, sel, _ = M.csa_query(q, t, iq, w, caches['dik'][0], caches['dk'][0], caches['dv'][0],
                                 caches['dwk'][0], caches['dwv'][0], m, k=1000)
    o2, l2 = M.hca_query(q, t, caches['dk'][0], caches['dv'][0], caches['dwk'][0], caches['dwv'][0], m)
    assert list(sel[:64]) == list(range(64)) and np.all(sel[64:] == -1)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(l1, l2)


def test_chunked_prefill_equals_one_shot():
    """P10: compressing a prefix in two chunks (the second starting at its own position)
    gives exactly the one-shot entries, and a query in the first chunk gets the same CSA
    and HCA results from the first chunk's caches alone as from the full caches, whose
    later entries and window rows it must not see."""
    g = np.random.default_rng(71)
    T, t0, D, dI, H, HI, m = 64, 32, 128, 64, 4, 4, 4
    rk, rv = g.standard_normal((1, T, D)).astype(np.float32), g.standard_normal((1, T, D)).astype(np.float32)
    ru = g.standard_normal((1, T, dI)).astype(np.float32)
    gate = g.standard_normal((1, T)).astype(np.float32)
    bias = (0.1 * g.standard_normal(m)).astype(np.float32)
    one = C.compress(rk, rv, gate, bias, 0, raw_ik=ru)
    a = C.compress(rk[:, :t0], rv[:, :t0], gate[:, :t0], bias, 0, raw_ik=ru[:, :t0])
    b = C.compress(rk[:, t0:], rv[:, t0:], gate[:, t0:], bias, t0, raw_ik=ru[:, t0:])
    for x, y, z in zip(one, a, b):
        assert np.array_equal(x, np.concatenate([y, z], axis=1))
    full = M.build_caches(rk, rv, gate, bias, 'f32', raw_ik=ru, ik_fmt='f32')
    half = M.build_caches(rk[:, :t0], rv[:, :t0], gate[:, :t0], bias, 'f32', raw_ik=ru[:, :t0], ik_fmt='f32')
    for t in (2, 3, 17, t0 - 1):
        q, iq = g.standard_normal((H, D)), g.standard_normal((HI, dI))
        w = g.uniform(size=HI)
        got = []
        for c in (full, half):
            got.append((M.csa_query(q, t, iq, w, c['dik'][0], c['dk'][0], c['dv'][0], c['dwk'][0], c['dwv'][0], m, 3,
                                    W=16),
                        M.hca_query(q, t, c['dk'][0], c['dv'][0], c['dwk'][0], c['dwv'][0], m, W=16)))
        for x, y in zip(got[0], got[1]):
            for u, v in zip(x, y):
                assert np.array_equal(np.asarray(u), np.asarray(v)), t


def test_visibility_rule():
    assert [I.n_visible(t, 4) for t in (0, 2, 3, 4, 7, 8)] == [0, 0, 1, 1, 2, 2]
    assert I.n_visible(1048575, 128) == 8192 and I.n_visible(1048575, 4) == 262144
    assert list(A.window_positions(5, 128)) == list(range(6))
    assert list(A.window_positions(300, 128)) == list(range(173, 301))


def test_page_constants_fixture():
    vals = {}
    for line in open(os.path.join(GOLDEN, 'page_constants.txt')):
        if line.strip() and not line.startswith('#'):
            name, val = line.split()[:2]
            vals[name] = int(val)
    assert vals['csa_ratio'] == 4 and vals['hca_ratio'] == 128 and vals['window'] == M.WINDOW
    assert vals['rope_dims'] == F.ROPE_DIM and vals['topk_pro'] == 1024 and vals['topk_flash'] == 512


# ------------------------------------------------------ compressor variants ----

def _rot_pair_loop(x, p, D, base=10000.0):
    """Rotate a raw row (list of floats) at position p with complex numbers, pair by pair."""
    out = list(x)
    for j in range(32):
        th = p * base ** (-(2 * j) / 64)
        z = complex(x[D - 64 + 2 * j], x[D - 64 + 2 * j + 1]) * complex(math.cos(th), math.sin(th))
        out[D - 64 + 2 * j], out[D - 64 + 2 * j + 1] = z.real, z.imag
    return out


def _variant_case(seed, B, T, D, dI, m, extra=0, channel=False):
    g = np.random.default_rng(seed)
    n = T + extra
    C = 2 * D + dI
    return dict(k=g.standard_normal((B, n, D)).astype(np.float32), v=g.standard_normal((B, n, D)).astype(np.float32),
                u=g.standard_normal((B, n, dI)).astype(np.float32),
                g=g.standard_normal((B, n, C) if channel else (B, n)).astype(np.float32))


def test_overlap_with_masked_previous_block_is_block():
    m, T, D, dI, pos0 = 4, 16, 128, 32, 8
    c = _variant_case(71, 2, T, D, dI, m, extra=m)
    beta = np.random.default_rng(72).normal(0, 0.1, m).astype(np.float32)
    bias = np.concatenate([np.full(m, -np.inf, np.float32), beta])
    got = C.compress_variant('overlap', c['k'], c['v'], c['g'], bias, pos0, raw_ik=c['u'])
    ref = C.compress(c['k'][:, m:], c['v'][:, m:], c['g'][:, m:], beta, pos0, raw_ik=c['u'][:, m:])
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= 1e-6 * np.abs(b).max()


def test_overlap_uniform_gate_is_window_mean_and_one_hot():
    m, T, D, dI = 4, 12, 128, 32
    c = _variant_case(73, 1, T, D, dI, m, extra=m)
    gate = np.zeros_like(c['g'])
    bias = np.zeros(2 * m, np.float32)
    # pos0 = 0: the first entry has no block before it (mean of its own 4 tokens)
    k, v, u = C.compress_variant('overlap', c['k'], c['v'], gate, bias, 0, raw_ik=c['u'])
    pos = np.arange(-m, T)
    kr = R.apply(c['k'].astype(np.float64), np.maximum(pos, 0)[None])
    assert np.allclose(v[0, 0], c['v'][0, m:2 * m].mean(0), atol=1e-6)
    assert np.allclose(k[0, 0], kr[0, m:2 * m].mean(0), atol=1e-6)
    for e in (1, 2):
        w = slice(e * m, e * m + 2 * m)
        assert np.allclose(v[0, e], c['v'][0, w].mean(0), atol=1e-6)
        assert np.allclose(u[0, e], c['u'][0, w].mean(0), atol=1e-6)
        assert np.allclose(k[0, e], kr[0, w].mean(0), atol=1e-6)
    # a one-hot gate on the second token of the previous block picks it (rotated at its own position)
    gate = np.zeros_like(c['g'])
    gate[0, m + 1] = 60.0                     # position 1, in the window of entry 1 (positions 0..7)
    k, v, _ = C.compress_variant('overlap', c['k'], c['v'], gate, bias, 0)
    assert np.allclose(v[0, 1], c['v'][0, m + 1], atol=1e-6)
    assert np.allclose(k[0, 1], R.apply(c['k'][0, m + 1].astype(np.float64), np.int64(1)), atol=1e-5)


def test_overlap_python_loop():
    m, T, D, dI, pos0 = 2, 6, 128, 32, 4
    c = _variant_case(74, 1, T, D, dI, m, extra=m)
    bias = np.random.default_rng(75).normal(0, 0.5, 2 * m).astype(np.float32)
    k, v, u = C.compress_variant('overlap', c['k'], c['v'], c['g'], bias, pos0, raw_ik=c['u'])
    for e in range(T // m):
        rows = [e * m + r for r in range(2 * m)]                       # window rows of entry e
        z = [float(c['g'][0, i]) + float(bias[r]) for r, i in enumerate(rows)]
        zmax = max(z)
        ex = [math.exp(zz - zmax) for zz in z]
        a = [x / sum(ex) for x in ex]
        krot = [_rot_pair_loop([float(x) for x in c['k'][0, i]], pos0 - m + i, D) for i in rows]
        for ch in (0, 77, 64 + 3, D - 1):
            assert abs(sum(a[r] * krot[r][ch] for r in range(2 * m)) - k[0, e, ch]) <= 1e-5
            assert abs(sum(a[r] * float(c['v'][0, rows[r], ch]) for r in range(2 * m)) - v[0, e, ch]) <= 1e-5
        assert abs(sum(a[r] * float(c['u'][0, rows[r], 5]) for r in range(2 * m)) - u[0, e, 5]) <= 1e-5


def test_rope_after_pool_reductions_and_complex_form():
    D, dI = 128, 32
    # m = 1: rotating before or after pooling one token is the same operation at the same position
    c = _variant_case(76, 2, 8, D, dI, 1)
    got = C.compress_variant('rope_after_pool', c['k'], c['v'], c['g'], np.zeros(1, np.float32), 40, raw_ik=c['u'])
    ref = C.compress(c['k'], c['v'], c['g'], np.zeros(1, np.float32), 40, raw_ik=c['u'])
    for a, b in zip(got, ref):
        assert np.array_equal(a, b)
    # m = 4: values and indexer keys as in the base reading; keys = e^{i theta p_last} x pooled pair
    m, pos0 = 4, 1000
    c = _variant_case(77, 2, 16, D, dI, m)
    beta = np.random.default_rng(78).normal(0, 0.1, m).astype(np.float32)
    k, v, u = C.compress_variant('rope_after_pool', c['k'], c['v'], c['g'], beta, pos0, raw_ik=c['u'])
    kb, vb, ub = C.compress(c['k'], c['v'], c['g'], beta, pos0, raw_ik=c['u'])
    assert np.array_equal(v, vb) and np.array_equal(u, ub)
    alpha = C.gate_weights(c['g'], beta)
    pooled = np.einsum('bem,bemc->bec', alpha, c['k'].astype(np.float64).reshape(2, 4, m, D))
    z = pooled[..., 64::2] + 1j * pooled[..., 65::2]
    theta = np.array([10000.0 ** (-(2 * j) / 64) for j in range(32)])
    last = pos0 + m - 1 + m * np.arange(4)
    zr = z * np.exp(1j * last[None, :, None] * theta[None, None, :])
    assert np.allclose(k[..., 64::2], zr.real, atol=1e-5) and np.allclose(k[..., 65::2], zr.imag, atol=1e-5)
    assert np.allclose(k[..., :64], pooled[..., :64], atol=1e-6)
    assert not np.allclose(k, kb, atol=1e-3)       # the placements differ


def test_channel_gate_reductions_one_hot_and_loop():
    m, T, D, dI, pos0 = 4, 8, 128, 32, 12
    c = _variant_case(79, 2, T, D, dI, m, channel=True)
    Cc = 2 * D + dI
    # equal gates in every channel: the base reading
    gs = c['g'][..., 0]
    beta = np.random.default_rng(80).normal(0, 0.1, m).astype(np.float32)
    got = C.compress_variant('channel_gate', c['k'], c['v'], np.repeat(gs[..., None], Cc, -1),
                             np.repeat(beta[:, None], Cc, -1), pos0, raw_ik=c['u'])
    ref = C.compress(c['k'], c['v'], gs, beta, pos0, raw_ik=c['u'])
    for a, b in zip(got, ref):
        assert np.abs(a - b).max() <= 1e-6 * np.abs(b).max()
    # one-hot per channel: channel ch of entry e takes token (ch % m) of its block
    gate = np.zeros((2, T, Cc), np.float32)
    for ch in range(Cc):
        gate[:, np.arange(T // m) * m + ch % m, ch] = 60.0
    k, v, u = C.compress_variant('channel_gate', c['k'], c['v'], gate, np.zeros((m, Cc), np.float32), pos0,
                                 raw_ik=c['u'])
    kr = R.apply(c['k'].astype(np.float64), (pos0 + np.arange(T))[None])
    for ch in (0, 5, 64, 101, 127):
        for e in range(T // m):
            assert abs(k[1, e, ch] - kr[1, e * m + ch % m, ch]) <= 1e-5
            assert abs(v[1, e, ch] - c['v'][1, e * m + (D + ch) % m, ch]) <= 1e-5
    assert abs(u[0, 1, 7] - c['u'][0, m + (2 * D + 7) % m, 7]) <= 1e-5
    # a plain loop on a few channels
    bias = np.random.default_rng(81).normal(0, 0.5, (m, Cc)).astype(np.float32)
    k, v, u = C.compress_variant('channel_gate', c['k'], c['v'], c['g'], bias, pos0, raw_ik=c['u'])
    for e in range(T // m):
        krot = [_rot_pair_loop([float(x) for x in c['k'][0, e * m + r]], pos0 + e * m + r, D) for r in range(m)]
        for ch, src, out, off in ((3, None, k, 0), (70, None, k, 0), (9, c['v'], v, D), (2, c['u'], u, 2 * D)):
            z = [float(c['g'][0, e * m + r, off + ch]) + float(bias[r, off + ch]) for r in range(m)]
            ex = [math.exp(zz - max(z)) for zz in z]
            vals = [krot[r][ch] for r in range(m)] if src is None else [float(src[0, e * m + r, ch]) for r in range(m)]
            assert abs(sum(x * y for x, y in zip(ex, vals)) / sum(ex) - out[0, e, ch]) <= 1e-5
