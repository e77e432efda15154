"""GPU parity at small sizes: every entry point against the oracle, through the C ABI.

Shapes span several tiles/chunks with ragged tails; edge cases cover empty and
short visibility, fewer visible entries than k, window shorter than W,
window-only layers, clustered winners (the exact fallback of the top-k merge)
and exact score ties.
"""

import numpy as np
import pytest
import torch

import long_context_attention_compress_amd as v4
import synth
from oracle import compress as OC
from oracle import formats as F
from oracle import indexer as OI
from oracle import model as OM
from tests.helpers import (TOL_BF16, TOL_F32, assert_close_rms, assert_codes_e4m3, assert_ik_rows, assert_kv_rows,
                           assert_topk, bf16_dev, dev, host_ik, host_kv, ik_store, kv_planes, kv_store, ring_rows)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- compress ----

# (1, 7, 63, 32): an odd number of window rows (the last pair of tokens has one) into a ring
# that keeps the last 32
@pytest.mark.parametrize('m,pos0,T,ring', [(4, 256, 64, 0), (1, 8, 40, 64), (1, 8, 200, 64), (1, 7, 63, 32),
                                           (128, 0, 384, 0)])
def test_compress_f32(m, pos0, T, ring):
    print(f'compress f32 m={m} pos0={pos0} T={T} ring={ring}', flush=True)
    raw = synth.raw_tokens(100 + m, 2, T, 128, m, 64, std=0.09, bf16=False)
    rows = (pos0 + T) // m if ring == 0 else ring
    ks = v4.KVStore.empty(2, rows, 128, v4.KV_F32, ring)
    vs = v4.KVStore.empty(2, rows, 128, v4.KV_F32, ring)
    iks = v4.IKStore.empty(2, (pos0 + T) // m, 64, v4.IK_F32)
    v4.csa_compress(dev(raw['gate']), dev(raw['pos_bias']), pos0, dev(raw['raw_k']), dev(raw['raw_v']), ks, vs,
                    dev(raw['raw_ik']), iks)
    torch.cuda.synchronize()
    k32, v32, u32 = OC.compress(raw['raw_k'], raw['raw_v'], raw['gate'], raw['pos_bias'], pos0, raw_ik=raw['raw_ik'])
    e0, ne = pos0 // m, T // m
    gk, gv, gu = host_kv(ks)['f32'], host_kv(vs)['f32'], host_ik(iks)['f32']
    if ring:
        keep = min(ne, ring)
        k32 = ring_rows(k32[:, ne - keep:], e0 + ne - keep, ring)
        v32 = ring_rows(v32[:, ne - keep:], e0 + ne - keep, ring)
        filled = [(e0 + i) % ring for i in range(ne - keep, ne)]
        assert_close_rms(gk[:, filled], k32[:, filled], 1e-6, 'k')
        assert_close_rms(gv[:, filled], v32[:, filled], 1e-6, 'v')
    else:
        assert_close_rms(gk[:, e0:], k32, 1e-6, 'k')
        assert_close_rms(gv[:, e0:], v32, 1e-6, 'v')
        assert np.all(gk[:, :e0] == 0)
    assert_close_rms(gu[:, e0:], u32, 1e-6, 'ik')


# (1, 4001, 201): an odd number of window rows at an odd position, the ring keeping the last 128
@pytest.mark.parametrize('m,pos0,T', [(4, 1024, 256), (1, 4000, 128), (1, 4001, 201), (128, 131072, 512)])
def test_compress_fp8_mxfp4(m, pos0, T):
    print(f'compress fp8 m={m} pos0={pos0} T={T}', flush=True)
    B = 2
    raw = synth.raw_tokens(200 + m, B, T, 192, m, 128, bf16=True)
    raw['raw_k'][0, 3, :] *= 30.0           # an outlier row: large scale
    raw['raw_v'][1, 5, :128] = 0.0          # a row whose E4M3 group is all zero when m == 1
    raw['raw_k'] = synth.to_bf16_values(raw['raw_k'])
    ring = 128 if m == 1 else 0
    rows = ring if ring else (pos0 + T) // m
    ks = v4.KVStore.empty(B, rows, 192, v4.KV_E4M3_BF16, ring)
    vs = v4.KVStore.empty(B, rows, 192, v4.KV_E4M3_BF16, ring)
    iks = v4.IKStore.empty(B, (pos0 + T) // m, 128, v4.IK_MXFP4)
    v4.csa_compress(dev(raw['gate']), dev(raw['pos_bias']), pos0, bf16_dev(raw['raw_k']), bf16_dev(raw['raw_v']),
                    ks, vs, bf16_dev(raw['raw_ik']), iks)
    torch.cuda.synchronize()
    k32, v32, u32 = OC.compress(raw['raw_k'], raw['raw_v'], raw['gate'], raw['pos_bias'], pos0, raw_ik=raw['raw_ik'])
    e0, ne = pos0 // m, T // m
    for name, x32, st in (('k', k32, ks), ('v', v32, vs)):
        g = host_kv(st)
        if ring:
            x32 = ring_rows(x32, e0, ring)
            sl = slice(None)
        else:
            sl = slice(e0, e0 + ne)
        codes, rope_bits, scale = F.kv_quantize(x32)
        assert np.array_equal(g['scale'][:, sl], scale), f'{name}: scales differ'
        assert np.array_equal(g['rope'][:, sl], rope_bits), f'{name}: bf16 RoPE dims differ'
        q = (x32[..., :128] / scale).astype(np.float32)
        assert_codes_e4m3(g['nope'][:, sl], codes, q, name)
    packed, scales = F.mxfp4_quantize(u32)
    gi = host_ik(iks)
    assert np.array_equal(gi['e8m0'][:, e0:e0 + ne], scales)
    assert np.array_equal(gi['e2m1'][:, e0:e0 + ne], packed)


@pytest.mark.parametrize('m,variant', [(1, 'block'), (4, 'block'), (128, 'block'), (4, 'overlap')])
def test_compress_wide_rows(m, variant):
    """Rows wider than one pair per lane: float32 K and V of dim 256 (192 no-RoPE dims, two
    pair iterations) and MXFP4 indexer keys of dim 192 (the second iteration half full), in
    BF16 activations, against the oracle: the float32 entries within float32 rounding, the
    MX scales and E2M1 codes exactly."""
    print(f'compress wide rows m={m} {variant}', flush=True)
    B, D, dI, pos0 = 2, 256, 192, 4 * 128
    T = 4 * m if m > 1 else 37
    extra = m if variant == 'overlap' else 0
    raw = synth.raw_tokens(300 + m, B, T + extra, D, m, dI, bf16=True, prefix=f'wide/{variant}')
    bias = raw['pos_bias'] if variant == 'block' else synth.normal(301, f'wide/b/{m}', (2 * m,), 0.1)
    rows = (pos0 + T) // m
    ks, vs = v4.KVStore.empty(B, rows, D, v4.KV_F32), v4.KVStore.empty(B, rows, D, v4.KV_F32)
    iks = v4.IKStore.empty(B, rows, dI, v4.IK_MXFP4)
    v4.csa_compress(dev(raw['gate']), dev(bias), pos0, bf16_dev(raw['raw_k']), bf16_dev(raw['raw_v']), ks, vs,
                    bf16_dev(raw['raw_ik']), iks, variant=v4.POOL_OVERLAP if variant == 'overlap' else v4.POOL_BLOCK)
    torch.cuda.synchronize()
    if variant == 'block':
        k32, v32, u32 = OC.compress(raw['raw_k'], raw['raw_v'], raw['gate'], bias, pos0, raw_ik=raw['raw_ik'])
    else:
        k32, v32, u32 = OC.compress_variant(variant, raw['raw_k'], raw['raw_v'], raw['gate'], bias, pos0,
                                            raw_ik=raw['raw_ik'])
    e0 = pos0 // m
    assert_close_rms(host_kv(ks)['f32'][:, e0:], k32, 1e-6, 'k')
    assert_close_rms(host_kv(vs)['f32'][:, e0:], v32, 1e-6, 'v')
    packed, scales = F.mxfp4_quantize(u32)
    gi = host_ik(iks)
    assert np.array_equal(gi['e8m0'][:, e0:], scales)
    assert np.array_equal(gi['e2m1'][:, e0:], packed)


@pytest.mark.parametrize('m', [1, 4, 128])
def test_compress_block_mode_device_positions(m):
    """Block mode: each batch element's block ends at a device position, raw inputs are a
    ring of 2m rows indexed by position. b0's block sits in the ring's second half (a large
    position), b1's position does not end a block (nothing written; for m = 1 every position
    does), b2 writes entry 0. Bitwise equal to the linear-mode call on the same rows."""
    B, D, dI = 3, 192, 128
    R = 2 * m
    raw = synth.raw_tokens(300 + m, B, R, D, m, dI if m == 4 else 0, bf16=True)
    ends = np.array([m * 1002 - 1, m * 500 + m // 2, m - 1], np.int64)
    ring = 128 if m == 1 else 0
    rows = 128 if m == 1 else 1100

    def stores():
        st = [v4.KVStore.empty(B, rows, D, ring=ring) for _ in range(2)]
        for x in st:
            x.nope.fill_(0x5A)
            x.rope.fill_(0x5A5A)
            x.scale.fill_(-7.0)
        ik = v4.IKStore.empty(B, rows, dI) if m == 4 else None
        if ik is not None:
            ik.e2m1.fill_(0xA5)
            ik.e8m0.fill_(0x33)
        return st[0], st[1], ik

    rk, rv = bf16_dev(raw['raw_k']), bf16_dev(raw['raw_v'])
    ru = bf16_dev(raw['raw_ik']) if m == 4 else None
    gate, bias = dev(raw['gate']), dev(raw['pos_bias'])
    k1, v1, i1 = stores()
    print(f'compress block mode m={m}', flush=True)
    v4.csa_compress(gate, bias, 0, rk, rv, k1, v1, ru, i1, block_end=dev(ends))
    k2, v2, i2 = stores()
    sl = lambda x, b: None if x is None else x[b:b + 1]
    for b in range(B):
        t = int(ends[b])
        if (t + 1) % m:
            continue
        first = t + 1 - m
        r0 = first % R
        one = lambda st: None if st is None else (
            v4.KVStore(st.fmt, st.dim, st.ring, nope=sl(st.nope, b), rope=sl(st.rope, b), scale=sl(st.scale, b))
            if isinstance(st, v4.KVStore) else v4.IKStore(st.fmt, st.dim, e2m1=sl(st.e2m1, b), e8m0=sl(st.e8m0, b)))
        v4.csa_compress(gate[b:b + 1, r0:r0 + m].contiguous(), bias, first, rk[b:b + 1, r0:r0 + m].contiguous(),
                        rv[b:b + 1, r0:r0 + m].contiguous(), one(k2), one(v2),
                        None if ru is None else ru[b:b + 1, r0:r0 + m].contiguous(), one(i2))
    torch.cuda.synchronize()
    for a, c in ((k1, k2), (v1, v2)):
        assert torch.equal(a.nope, c.nope) and torch.equal(a.rope, c.rope)
        assert torch.equal(a.scale.view(torch.int32), c.scale.view(torch.int32))
    if m == 4:
        assert torch.equal(i1.e2m1, i2.e2m1) and torch.equal(i1.e8m0, i2.e8m0)
    if m > 1:
        assert torch.all(k1.nope[1] == 0x5A), 'a position inside a block wrote an entry'


VARIANT_CASES = [('overlap', 4, 0), ('overlap', 4, 1024), ('overlap', 128, 131072), ('rope_after_pool', 4, 1000),
                 ('rope_after_pool', 128, 131072), ('channel_gate', 4, 1024), ('channel_gate', 128, 0)]


@pytest.mark.parametrize('variant,m,pos0', VARIANT_CASES)
def test_compress_variants(variant, m, pos0):
    """Each compressor variant against the oracle's reading of it, every plane of K, V and
    (for m = 4) the MXFP4 indexer key: overlapping windows (including the first entry, whose
    block before does not exist), RoPE after pooling, per-channel gates."""
    B, D, dI = 2, 192, 128
    T = 8 * m
    enum = {'overlap': v4.POOL_OVERLAP, 'rope_after_pool': v4.POOL_ROPE_AFTER, 'channel_gate': v4.POOL_CHANNEL_GATE}
    with_ik = m == 4
    extra = m if variant == 'overlap' else 0
    raw = synth.raw_tokens(400 + m, B, T + extra, D, m, dI if with_ik else 0, bf16=True, prefix=f'var/{variant}')
    C = 2 * D + (dI if with_ik else 0)
    if variant == 'channel_gate':
        gate = synth.normal(401, f'var/cg/{m}', (B, T, C))
        bias = synth.normal(402, f'var/cb/{m}', (m, C), 0.1)
    else:
        gate = raw['gate']
        bias = synth.normal(403, f'var/b/{variant}/{m}', (2 * m if variant == 'overlap' else m,), 0.1)
    rows = (pos0 + T) // m
    ks, vs = v4.KVStore.empty(B, rows, D), v4.KVStore.empty(B, rows, D)
    iks = v4.IKStore.empty(B, rows, dI) if with_ik else None
    print(f'compress variant {variant} m={m} pos0={pos0}', flush=True)
    v4.csa_compress(dev(gate), dev(bias), pos0, bf16_dev(raw['raw_k']), bf16_dev(raw['raw_v']), ks, vs,
                    bf16_dev(raw['raw_ik']) if with_ik else None, iks, variant=enum[variant])
    torch.cuda.synchronize()
    k32, v32, u32 = OC.compress_variant(variant, raw['raw_k'], raw['raw_v'], gate, bias, pos0,
                                        raw_ik=raw['raw_ik'] if with_ik else None)
    new = np.arange(pos0 // m, pos0 // m + T // m)
    for b in range(B):
        n = assert_kv_rows(*kv_planes(ks, b, new), k32[b], f'{variant} K b{b}')
        n += assert_kv_rows(*kv_planes(vs, b, new), v32[b], f'{variant} V b{b}')
        if with_ik:
            n += assert_ik_rows(iks.e2m1[b, new[0]:].cpu().numpy(), iks.e8m0[b, new[0]:].cpu().numpy(), u32[b],
                                f'{variant} indexer key b{b}')
        print(f'[planes] {variant} m={m} b{b}: {n} boundary differences', flush=True)


def test_compress_overlap_block_mode():
    """Overlapping windows in block mode: a raw ring of 2m rows indexed by position, the
    block ending at a device position; b0 at a large position, b1 the first entry (no
    block before it), equal bitwise to the linear call on the same window."""
    B, D, dI, m = 2, 192, 128, 4
    R = 2 * m
    raw = synth.raw_tokens(410, B, R, D, m, dI, bf16=True, prefix='var/ring')
    bias = dev(synth.normal(411, 'var/ring/b', (2 * m,), 0.1))
    ends = np.array([4 * 2501 - 1, m - 1], np.int64)
    rows = 2600
    st = lambda: (v4.KVStore.empty(B, rows, D), v4.KVStore.empty(B, rows, D), v4.IKStore.empty(B, rows, dI))
    k1, v1, i1 = st()
    rk, rv, ru, g = bf16_dev(raw['raw_k']), bf16_dev(raw['raw_v']), bf16_dev(raw['raw_ik']), dev(raw['gate'])
    v4.csa_compress(g, bias, 0, rk, rv, k1, v1, ru, i1, block_end=dev(ends), variant=v4.POOL_OVERLAP)
    k2, v2, i2 = st()
    for b in range(B):
        first = int(ends[b]) + 1 - m
        order = [(first - m + r) % R for r in range(2 * m)]          # window rows by position
        one = lambda x: x[b:b + 1]
        sub = lambda t: t[b:b + 1][:, order].contiguous()
        v4.csa_compress(sub(g), bias, first, sub(rk), sub(rv),
                        v4.KVStore(k2.fmt, D, 0, nope=one(k2.nope), rope=one(k2.rope), scale=one(k2.scale)),
                        v4.KVStore(v2.fmt, D, 0, nope=one(v2.nope), rope=one(v2.rope), scale=one(v2.scale)),
                        sub(ru), v4.IKStore(i2.fmt, dI, e2m1=one(i2.e2m1), e8m0=one(i2.e8m0)),
                        variant=v4.POOL_OVERLAP)
    torch.cuda.synchronize()
    for a, c in ((k1, k2), (v1, v2)):
        assert torch.equal(a.nope, c.nope) and torch.equal(a.rope, c.rope)
        assert torch.equal(a.scale.view(torch.int32), c.scale.view(torch.int32))
    assert torch.equal(i1.e2m1, i2.e2m1) and torch.equal(i1.e8m0, i2.e8m0)


# ---------------------------------------------------------------- index ----

def _index_case_mx(seed, B, rows, q_pos, k, m=4, cluster=None, ties=False):
    H, dI = 64, 128
    g = np.random.default_rng(seed)
    keys = synth.normal(seed, 'ik', (B, rows, dI))
    iq = synth.normal(seed, 'iq', (B, q_pos.shape[1], H, dI))
    w = synth.uniform(seed, 'w', (B, q_pos.shape[1], H))
    if cluster is not None:          # winners packed into one chunk: exercises the exact fallback
        b, lo, n = cluster
        d = (w[b, 0][:, None] * iq[b, 0]).sum(0)
        keys[b, lo:lo + n] = 6.0 * np.sqrt(dI) * d / np.linalg.norm(d) + 0.05 * g.standard_normal((n, dI))
    if ties:                         # many exact duplicates of a few keys
        keys[:, 1::3] = keys[:, 0:1]
    packed, sc = F.mxfp4_quantize(keys)
    ip, isc = F.mxfp4_quantize(iq)
    return dict(packed=packed, sc=sc, ip=ip, isc=isc, w=w, q_pos=q_pos, k=k, m=m,
                dkeys=F.mxfp4_dequantize(packed, sc), diq=F.mxfp4_dequantize(ip, isc))


def _run_index(c, fmt='mx'):
    if fmt == 'mx':
        store = v4.IKStore(v4.IK_MXFP4, 128, e2m1=dev(c['packed']), e8m0=dev(c['sc']))
        iq, iqs = dev(c['ip']), dev(c['isc'])
    else:
        store = v4.IKStore(v4.IK_F32, c['keys'].shape[-1], f32=dev(c['keys']))
        iq, iqs = dev(c['iq']), None
    B, Tq = c['q_pos'].shape
    score = torch.zeros(B, Tq, c['k'], dtype=torch.float32, device='cuda')
    idx = v4.lightning_index_topk(dev(c['q_pos']), iq, dev(c['w']), store, c['k'], c['m'], iq_scale=iqs,
                                  out_score=score)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), score.cpu().numpy()


def _same_bits(a, b):
    """Bitwise equality of float arrays (NaN scores included)."""
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def _check_index(c, idx, score, dkeys, diq):
    B, Tq = c['q_pos'].shape
    rows = dkeys.shape[1]
    for b in range(B):
        for i in range(Tq):
            t = int(c['q_pos'][b, i])
            n_vis = OI.n_visible(t, c['m'], rows) if t >= 0 else 0
            s = OI.index_scores(diq[b, i], c['w'][b, i], dkeys[b, :n_vis])
            assert_topk(idx[b, i], s, n_vis, c['k'], f'b{b} i{i} t{t}')
            kk = min(c['k'], n_vis)
            sel = idx[b, i, :kk]
            ref = s[sel].astype(np.float32)
            assert np.allclose(score[b, i, :kk], ref, rtol=2e-6, atol=1e-30, equal_nan=True), f'scores b{b} i{i}'
            assert np.all(score[b, i, kk:] == 0)


def test_index_mxfp4_shapes_and_edges():
    q_pos = np.array([[19999, 12345], [7, 3000], [2047, -1], [2, 1]], np.int64)
    c = _index_case_mx(1, 4, 5000, q_pos, 512)
    print('index mxfp4 edges', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, c['dkeys'], c['diq'])


@pytest.mark.parametrize('rows,k', [(1025, 512), (4096, 1024), (4097, 2048), (8193, 1024)])
def test_index_mxfp4_multi_query_chunk_boundaries(rows, k):
    """Several queries per sequence over more than 1,024 entries: the layout's chunk is four
    1,024-entry sub-chunks with one candidate emission each (one workgroup per chunk). Entry
    counts just past a sub-chunk, at and just past a chunk, and past two chunks; queries that
    see every entry, part of a chunk, or almost nothing; k up to 2,048, where a chunk's share
    is capped by its region. Checked against the oracle, and bitwise against one call per
    query (the one-chunk scorer)."""
    n = rows * 4
    q_pos = np.array([[n - 1, (rows // 2) * 4 + 1, 4 * 3 - 1],
                      [(rows - 1) * 4 - 1, 4 * 1030 - 1, -1]], np.int64)
    c = _index_case_mx(43 + rows, 2, rows, q_pos, k)
    print(f'index mxfp4, 3 queries per sequence over {rows} entries, k {k}', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, c['dkeys'], c['diq'])
    for i in range(q_pos.shape[1]):
        ci = dict(c, q_pos=c['q_pos'][:, i:i + 1], ip=c['ip'][:, i:i + 1], isc=c['isc'][:, i:i + 1],
                  w=c['w'][:, i:i + 1])
        idx1, score1 = _run_index(ci)
        assert np.array_equal(idx1[:, 0], idx[:, i]) and _same_bits(score1[:, 0], score[:, i]), f'query {i}'


@pytest.mark.parametrize('k', [64, 1024])
def test_index_mxfp4_merge_widths(k):
    """The merge runs 512 threads per query from 512 queries per call and 1,024 below:
    600 queries made of 6 patterns (same query rows and positions) against a call with
    the 6 alone, bitwise (ids and scores), and the 6 against the oracle."""
    rows, P, R = 20000, 6, 100
    q_pos = np.array([[rows * 4 - 1, 70001, 40003, 9000, 4095, 130]], np.int64)
    c = _index_case_mx(61 + k, 1, rows, q_pos, k)
    print(f'index merge widths, k {k}', flush=True)
    idx6, score6 = _run_index(c)
    _check_index(c, idx6, score6, c['dkeys'], c['diq'])
    pat = np.arange(P * R) % P
    cw = dict(c, q_pos=c['q_pos'][:, pat], ip=c['ip'][:, pat], isc=c['isc'][:, pat], w=c['w'][:, pat])
    idx, score = _run_index(cw)
    for j in range(P * R):
        assert np.array_equal(idx[0, j], idx6[0, pat[j]]), f'ids of query {j}'
        assert _same_bits(score[0, j], score6[0, pat[j]]), f'scores of query {j}'


def test_index_mxfp4_clustered_winners_and_ties():
    q_pos = np.array([[40000 * 4 - 1], [20000]], np.int64)
    c = _index_case_mx(2, 2, 40000, q_pos, 1024, cluster=(0, 3000, 1500), ties=True)
    print('index mxfp4 clustered', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, c['dkeys'], c['diq'])


def test_index_mxfp4_exponent_extremes():
    """Exponent bytes that send tiles to the exact pass of the scorer: keys scaled by
    2^84 with a query head scaled by 2^34 (no overflow, but the bound on |q.k| no
    longer rules it out), NaN key exponents (0xFF: those keys score NaN and rank
    last) and, in batch 1, a NaN query exponent (every tile exact; every score NaN,
    so the selection is the lowest ids)."""
    rows = 6000
    q_pos = np.array([[rows * 4 - 1], [rows * 4 - 1]], np.int64)
    c = _index_case_mx(5, 2, rows, q_pos, 256)
    sc, isc = c['sc'].copy(), c['isc'].copy()
    sc[:, ::97] += 84                     # rows 0, 97, ...: x 2^84
    sc[:, 5::211, 2] = 0xFF               # NaN in one 32-dim block
    isc[0, 0, 3] += 34                    # batch 0: head 3 x 2^34
    isc[1, 0, 7, 1] = 0xFF                # batch 1: NaN query block -> every tile exact
    c['sc'], c['isc'] = sc, isc
    dkeys, diq = F.mxfp4_dequantize(c['packed'], sc), F.mxfp4_dequantize(c['ip'], isc)
    for b in range(2):
        s = OI.index_scores(diq[b, 0], c['w'][b, 0], dkeys[b])
        assert not np.isinf(s.astype(np.float32)).any(), 'the case must not overflow float32'
    assert np.isnan(OI.index_scores(diq[1, 0], c['w'][1, 0], dkeys[1])).all()
    print('index mxfp4 exponent extremes', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, dkeys, diq)


def test_index_mxfp4_many_queries_per_sequence():
    """Thirteen queries per sequence in one call: positions in and out of order, queries
    that see nothing or only part of a chunk, one query whose scaled head sends its tiles
    to the exact pass while its neighbours take the fast form, and one with a NaN query
    exponent (every tile exact). Checked against the oracle, and bitwise against one call
    per query (no state leaks between the queries of a call)."""
    rows, Tq = 6000, 13
    g = np.random.default_rng(21)
    q_pos = np.stack([np.arange(rows * 4 - Tq, rows * 4),
                      np.sort(g.integers(0, rows * 4, Tq))[::-1]]).astype(np.int64)
    q_pos[1, 5], q_pos[1, 9], q_pos[1, 12] = -1, 2, 4095
    c = _index_case_mx(21, 2, rows, q_pos, 512)
    sc, isc = c['sc'].copy(), c['isc'].copy()
    sc[:, ::97] += 84                     # rows 0, 97, ...: x 2^84
    isc[1, 3, 3] += 34                    # query 3 of batch 1: head 3 x 2^34 -> exact pass
    isc[0, 6, 9, 2] = 0xFF                # query 6 of batch 0: a NaN block -> every tile exact
    c['sc'], c['isc'] = sc, isc
    dkeys, diq = F.mxfp4_dequantize(c['packed'], sc), F.mxfp4_dequantize(c['ip'], isc)
    print('index mxfp4 multi-query', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, dkeys, diq)
    for i in range(Tq):
        ci = dict(c, q_pos=c['q_pos'][:, i:i + 1], ip=c['ip'][:, i:i + 1], isc=c['isc'][:, i:i + 1],
                  w=c['w'][:, i:i + 1])
        idx1, score1 = _run_index(ci)
        assert np.array_equal(idx1[:, 0], idx[:, i]) and _same_bits(score1[:, 0], score[:, i]), f'query {i}'


def test_index_mxfp4_tokens_sharing_a_large_key_set():
    """Six tokens per sequence over 70,000 entries (4.8 MB of keys, more than an XCD's
    L2), as when draft tokens are decoded together at a long context: tokens that see
    all, part or none of the keys, and one token whose scaled head takes the exact pass.
    Checked against the oracle, and bitwise against one call per token (the one-chunk
    scorer)."""
    rows, Tq = 70000, 6
    q_pos = np.array([[rows * 4 - 1 - i for i in range(Tq)],
                      [rows * 4 - 1, 123456, -1, 2, 4095, 200001]], np.int64)
    c = _index_case_mx(41, 2, rows, q_pos, 1024)
    sc, isc = c['sc'].copy(), c['isc'].copy()
    sc[:, ::997] += 84                    # every 997th row x 2^84
    isc[1, 1, 3] += 34                    # token 1 of batch 1: head 3 x 2^34 -> exact pass
    c['sc'], c['isc'] = sc, isc
    dkeys, diq = F.mxfp4_dequantize(c['packed'], sc), F.mxfp4_dequantize(c['ip'], isc)
    print('index mxfp4, six tokens per sequence over 70000 entries', flush=True)
    idx, score = _run_index(c)
    _check_index(c, idx, score, dkeys, diq)
    for i in range(Tq):
        ci = dict(c, q_pos=c['q_pos'][:, i:i + 1], ip=c['ip'][:, i:i + 1], isc=c['isc'][:, i:i + 1],
                  w=c['w'][:, i:i + 1])
        idx1, score1 = _run_index(ci)
        assert np.array_equal(idx1[:, 0], idx[:, i]) and _same_bits(score1[:, 0], score[:, i]), f'token {i}'


def test_index_mxfp4_repeat_is_bitwise_identical():
    q_pos = np.array([[12000 * 4 - 1]], np.int64)
    c = _index_case_mx(3, 1, 12000, q_pos, 256)
    a = _run_index(c)
    b = _run_index(c)
    assert np.array_equal(a[0], b[0]) and _same_bits(a[1], b[1])


def test_index_f32_small():
    seed, B, Tq, rows, H, dI = 4, 1, 16, 1024, 4, 64
    keys = synth.normal(seed, 'k', (B, rows, dI), 0.125)
    iq = synth.normal(seed, 'q', (B, Tq, H, dI), 0.125)
    w = synth.uniform(seed, 'w', (B, Tq, H))
    q_pos = np.arange(4096 - Tq, 4096, dtype=np.int64)[None]
    q_pos[0, 0] = 9            # 2 visible entries
    q_pos[0, 1] = 300          # 75 visible: more than k
    c = dict(keys=keys, iq=iq, w=w, q_pos=q_pos, k=64, m=4)
    idx, score = _run_index(c, 'f32')
    _check_index(c, idx, score, keys.astype(np.float64), iq.astype(np.float64))


# ------------------------------------------------------------ attention ----

def _attn_case(seed, B, Tq, H, D, rows, q_pos, fmt, W=128, ring=0):
    outl = 0.01 if fmt == 'fp8' else 0.0
    std = 1.0 if fmt == 'fp8' else 0.09
    ent_k = synth.normal(seed, 'ek', (B, rows, D), std, outl)
    ent_v = synth.normal(seed, 'ev', (B, rows, D), std, outl)
    # raw window rows: a linear store of every position up to the latest query
    # (ring == 0), or a ring holding the last `ring` positions
    tmax = int(q_pos.max())
    first = max(0, tmax - ring + 1) if ring else 0
    win_k = synth.normal(seed, 'wk', (B, tmax - first + 1, D), std, outl)
    win_v = synth.normal(seed, 'wv', (B, tmax - first + 1, D), std, outl)
    q = synth.normal(seed, 'q', (B, Tq, H, D), std, outl)
    if fmt == 'fp8':
        q = synth.to_bf16_values(q)
    kvf = 'f32' if fmt == 'f32' else 'e4m3_bf16'
    enc = {n: OC.encode_kv(x, kvf) for n, x in (('ek', ent_k), ('ev', ent_v), ('wk', win_k), ('wv', win_v))}
    dec = {n: OC.decode_kv(e) for n, e in enc.items()}
    ring_enc = {}
    for n in ('wk', 'wv'):
        ring_enc[n] = {pk: (ring_rows(pv, first, ring) if ring else pv) for pk, pv in enc[n].items()}
    return dict(q=q, q_pos=q_pos, enc=enc, dec=dec, ring_enc=ring_enc, first=first, W=W, ring=ring, fmt=fmt,
                H=H, D=D)


def _stores(c):
    return (kv_store(c['enc']['ek']), kv_store(c['enc']['ev']), kv_store(c['ring_enc']['wk'], c['ring']),
            kv_store(c['ring_enc']['wv'], c['ring']))


def _qdev(c):
    return bf16_dev(c['q']) if c['fmt'] == 'fp8' else dev(c['q'])


def _oracle_attn(c, b, i, ids):
    t = int(c['q_pos'][b, i])
    return OM.A.attend_query(c['q'][b, i], t, ids, c['dec']['ek'][b], c['dec']['ev'][b], c['dec']['wk'][b],
                             c['dec']['wv'][b], c['W'], win_first=c['first'])


@pytest.mark.parametrize('fmt', ['f32', 'fp8'])
def test_attn_sparse(fmt):
    B, Tq, rows, k = 2, 3, 1000, 192
    H, D = (16, 128) if fmt == 'f32' else (64, 192)
    q_pos = np.array([[3999, 3998, 3900], [3999, 3000, 3999]], np.int64)
    c = _attn_case(10, B, Tq, H, D, rows, q_pos, fmt)
    g = np.random.default_rng(11)
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for i in range(Tq):
            n = [k, 150, 37][i]
            idx[b, i, :n] = np.sort(g.choice(rows, n, replace=False))
    idx[1, 2, 5] = rows + 7           # out-of-range ids are skipped
    ek, ev, wk, wv = _stores(c)
    lse = torch.zeros(B, Tq, H, dtype=torch.float32, device='cuda')
    print(f'attn sparse {fmt}', flush=True)
    o = v4.sparse_window_attn(_qdev(c), dev(q_pos), ek, ev, 4, wk, wv, c['W'], dev(idx), lse=lse)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    tol = TOL_F32 if fmt == 'f32' else TOL_BF16
    for b in range(B):
        for i in range(Tq):
            ids = idx[b, i]
            ids = ids[(ids >= 0) & (ids < rows)]
            ro, rl = _oracle_attn(c, b, i, ids)
            assert_close_rms(o[b, i], ro, tol, f'o b{b} i{i}')
            assert np.allclose(lse[b, i], rl, atol=1e-4 if fmt == 'f32' else 2e-2), f'lse b{b} i{i}'


@pytest.mark.parametrize('fmt', ['f32', 'fp8'])
@pytest.mark.parametrize('override', [-1, 0, 100])
def test_attn_dense(fmt, override):
    B, Tq, rows, m = 2, 2, 700, 4
    H, D = (16, 128) if fmt == 'f32' else (64, 192)
    q_pos = np.array([[2799, 60], [1234, 2799]], np.int64)    # 60: window shorter than W, 15 entries
    c = _attn_case(12, B, Tq, H, D, rows, q_pos, fmt)
    ek, ev, wk, wv = _stores(c)
    print(f'attn dense {fmt} override={override}', flush=True)
    o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'], n_entries_override=override)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    tol = TOL_F32 if fmt == 'f32' else TOL_BF16
    for b in range(B):
        for i in range(Tq):
            t = int(q_pos[b, i])
            n = min((t + 1) // m, rows)
            if override >= 0:
                n = min(n, override)
            ro, _ = _oracle_attn(c, b, i, np.arange(n))
            assert_close_rms(o[b, i], ro, tol, f'o b{b} i{i}')


# Positions past 2^31 take the 64-bit divisions of the key-list geometry (the
# entry count (t + 1) // m and the window's ring slot); a large m keeps the
# entry store small while the division still decides the count: with
# m = 8,388,617, t + 1 = 256 m is the first position past 2^31 that sees 256
# entries, and t + 1 = 255 m (below 2^31) a boundary of the fast path.
BIG_M = 8388617


@pytest.mark.parametrize('q_pos', [[256 * BIG_M - 2, 256 * BIG_M - 1], [255 * BIG_M - 2, 255 * BIG_M - 1]])
def test_attn_positions_past_2_31(q_pos):
    B, Tq, H, D, rows = 1, 2, 64, 192, 300
    q_pos = np.array([q_pos], np.int64)
    c = _attn_case(15, B, Tq, H, D, rows, q_pos, 'fp8', ring=200)
    ek, ev, wk, wv = _stores(c)
    print(f'attn positions {q_pos.tolist()}', flush=True)
    o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, BIG_M, wk, wv, c['W'])
    g = np.random.default_rng(16)
    k = 64
    idx = np.stack([np.sort(g.choice(rows, k, replace=False)) for _ in range(Tq)])[None].astype(np.int32)
    os_ = v4.sparse_window_attn(_qdev(c), dev(q_pos), ek, ev, 4, wk, wv, c['W'], dev(idx))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    os_ = os_.float().cpu().numpy()
    for i in range(Tq):
        t = int(q_pos[0, i])
        n = min((t + 1) // BIG_M, rows)
        assert n in (254, 255, 256)
        ro, _ = _oracle_attn(c, 0, i, np.arange(n))
        assert_close_rms(o[0, i], ro, TOL_BF16, f'dense o i{i}')
        ro, _ = _oracle_attn(c, 0, i, idx[0, i])
        assert_close_rms(os_[0, i], ro, TOL_BF16, f'sparse o i{i}')


def test_more_queries_than_one_launch_row():
    """70,000 queries in one call, more than one launch takes along the query axis, so
    the library splits it: the index and dense attention, with query rows drawn from 64
    patterns and random positions, checked against the oracle on queries on both sides
    of each split point."""
    NQ, P, rows, m = 70000, 64, 300, 4
    g = np.random.default_rng(31)
    pat = g.integers(0, P, NQ)
    q_pos = g.integers(0, rows * m, NQ).astype(np.int64)[None]
    S = np.array([0, 1, 65533, 65534, 65535, 65536, 69999] + list(g.integers(0, NQ, 6)))

    base = _index_case_mx(31, 1, rows, np.zeros((1, P), np.int64), 16)
    c = dict(base, ip=base['ip'][:, pat], isc=base['isc'][:, pat], w=base['w'][:, pat], q_pos=q_pos)
    print('index, 70000 queries', flush=True)
    idx, score = _run_index(c)
    cs = dict(c, q_pos=q_pos[:, S], w=c['w'][:, S])
    _check_index(cs, idx[:, S], score[:, S], base['dkeys'], base['diq'][:, pat[S]])

    H, D = 16, 192
    a = _attn_case(32, 1, P, H, D, rows, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(a)
    qd = bf16_dev(a['q'])[:, torch.from_numpy(pat).cuda()].contiguous()
    print('dense attention, 70000 queries', flush=True)
    o = v4.hca_attn(qd, dev(q_pos), ek, ev, m, wk, wv, a['W'])
    o = o[:, torch.from_numpy(S).cuda()].float().cpu().numpy()
    for j, s in enumerate(S):
        t = int(q_pos[0, s])
        ro, _ = OM.A.attend_query(a['q'][0, pat[s]], t, np.arange(min((t + 1) // m, rows)), a['dec']['ek'][0],
                                  a['dec']['ev'][0], a['dec']['wk'][0], a['dec']['wv'][0], a['W'],
                                  win_first=a['first'])
        assert_close_rms(o[0, j], ro, TOL_BF16, f'o query {s}')


def test_attn_many_query_head_pairs_combine():
    """Four tokens per sequence, B = 4, 64 heads: 1,024 query-head pairs (at least 512), where the split
    partials are merged by one thread per output dimension; sparse and dense against the
    oracle."""
    B, Tq, rows, m, H, D, k = 4, 4, 1500, 4, 64, 192, 256
    q_pos = np.array([[rows * m - 1 - i for i in range(Tq)]] * B, np.int64)
    q_pos[2, 1] = 777
    c = _attn_case(71, B, Tq, H, D, rows, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(c)
    g = np.random.default_rng(72)
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        for i in range(Tq):
            nv = min((int(q_pos[b, i]) + 1) // m, rows)
            sel = np.sort(g.choice(nv, min(k, nv), replace=False))
            idx[b, i, :len(sel)] = sel
    print('combine with 1024 query-head pairs', flush=True)
    for name in ('sparse', 'dense'):
        if name == 'sparse':
            o = v4.sparse_window_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'], dev(idx))
        else:
            o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'])
        torch.cuda.synchronize()
        o = o.float().cpu().numpy()
        for b in range(B):
            for i in range(Tq):
                t = int(q_pos[b, i])
                ids = idx[b, i][idx[b, i] >= 0] if name == 'sparse' else np.arange(min((t + 1) // m, rows))
                ro, _ = _oracle_attn(c, b, i, ids)
                assert_close_rms(o[b, i], ro, TOL_BF16, f'{name} b{b} i{i}')


@pytest.mark.parametrize('n_split', [16, 17, 48, 49, 64, 65])
def test_attn_combine_split_counts(n_split):
    """Sparse calls whose key list (k id slots + W window rows = 32 n keys, one tile per
    split) gives n splits: the one-thread-per-dim combine at each of its load counts
    (16, 32, 48, 64 splits: 16 and 17, 48 and 49, 64) and the grouped combine above 64
    splits. The last 64 id slots are empty, so whole splits have no key (max -inf, sum 0);
    outputs and log-sum-exps against the oracle."""
    B, Tq, rows, m, H, D, W = 2, 1, 3000, 4, 64, 192, 128
    k = 32 * n_split - W
    q_pos = np.array([[rows * m - 1], [rows * m - 1 - 9]], np.int64)
    c = _attn_case(81 + n_split, B, Tq, H, D, rows, q_pos, 'fp8', W=W)
    ek, ev, wk, wv = _stores(c)
    g = np.random.default_rng(82 + n_split)
    idx = np.full((B, Tq, k), -1, np.int32)
    for b in range(B):
        idx[b, 0, :k - 64] = np.sort(g.choice(rows, k - 64, replace=False))
    lse = torch.zeros(B, Tq, H, dtype=torch.float32, device='cuda')
    print(f'combine over {n_split} splits', flush=True)
    o = v4.sparse_window_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, W, dev(idx), lse=lse)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    for b in range(B):
        ids = idx[b, 0][idx[b, 0] >= 0]
        ro, rl = _oracle_attn(c, b, 0, ids)
        assert_close_rms(o[b, 0], ro, TOL_BF16, f'o b{b}')
        assert np.allclose(lse[b, 0], rl, atol=2e-2), f'lse b{b}'


@pytest.mark.parametrize('Tq', [3, 70])
def test_attn_dense_long_list(Tq):
    """A key list of more than 4096 keys with the window (two key streams per
    workgroup), with queries that see all entries, part of them, and almost none
    (ragged and empty tiles in both streams); 3 queries (many splits each) and 70
    (fewer splits per query)."""
    B, rows, m = 1, 6000, 4
    H, D = 64, 192
    base = [rows * m - 1, 9001, 130]
    q_pos = np.array([[base[i % 3] - 7 * (i // 3) for i in range(Tq)]], np.int64)
    c = _attn_case(13, B, Tq, H, D, rows, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(c)
    print(f'attn dense long list, {Tq} queries', flush=True)
    o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'])
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for i in sorted({0, 1, 2, Tq - 1, Tq // 2}):
        t = int(q_pos[0, i])
        n = min((t + 1) // m, rows)
        ro, _ = _oracle_attn(c, 0, i, np.arange(n))
        assert_close_rms(o[0, i], ro, TOL_BF16, f'o i{i} t{t}')


@pytest.mark.parametrize('t_last', [128, 1000])
def test_attn_window_only_ring(t_last):
    # one query per batch element at the ring's newest position, plus early positions
    B, Tq, H, D = 1, 2, 64, 192
    q_pos = np.array([[t_last - 1, t_last]], np.int64)
    c = _attn_case(13, B, Tq, H, D, 8, q_pos, 'fp8', ring=129)
    ek, ev, wk, wv = _stores(c)
    o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, 4, wk, wv, 128, n_entries_override=0)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for i in range(Tq):
        ro, _ = _oracle_attn(c, 0, i, np.zeros(0, np.int64))
        assert_close_rms(o[0, i], ro, TOL_BF16, f'o i{i}')


def test_attn_window_only_first_positions():
    B, Tq, H, D = 1, 4, 64, 192
    q_pos = np.array([[0, 1, 127, 128]], np.int64)
    c = _attn_case(14, B, Tq, H, D, 8, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(c)
    o = v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, 4, wk, wv, 128, n_entries_override=0)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for i in range(Tq):
        ro, _ = _oracle_attn(c, 0, i, np.zeros(0, np.int64))
        assert_close_rms(o[0, i], ro, TOL_BF16, f'o i{i}')


def _batch_view(st, b):
    return v4.KVStore(st.fmt, st.dim, st.ring, nope=st.nope[b:b + 1], rope=st.rope[b:b + 1],
                      scale=st.scale[b:b + 1])


# (kind, B, rows, k, q positions, window ring): the fused append's key in a
# sparse split (linear window store and ring), in a short linear window
# (t = 60), in a two-stream dense workgroup, and in a window-only layer.
# Queries of one case that use a ring share their position.
APPEND_CASES = [
    ('sparse', 2, 1000, 192, [3999, 3001], 0),
    ('sparse', 2, 1000, 192, [3999, 3999], 200),
    ('dense', 2, 700, 0, [2799, 60], 0),
    ('dense', 1, 6000, 0, [23999], 130),
    ('window', 1, 8, 0, [1000], 129),
]


@pytest.mark.parametrize('case', range(len(APPEND_CASES)))
def test_attn_fused_window_append(case):
    """Attention with the fused window append against csa_compress (m = 1) then
    attention without it: bitwise-equal window stores and outputs. The appended
    row also equals the oracle's m = 1 compression of the raw row, and the
    output matches the oracle over the updated window."""
    kind, B, rows, k, pos, ring = APPEND_CASES[case]
    m = 4
    q_pos = np.array(pos, np.int64).reshape(B, 1)
    c = _attn_case(40 + case, B, 1, 64, 192, rows, q_pos, 'fp8', ring=ring)
    raw_k = synth.to_bf16_values(synth.normal(40 + case, 'app/k', (B, 1, 192), 1.0, 0.01))
    raw_v = synth.to_bf16_values(synth.normal(40 + case, 'app/v', (B, 1, 192), 1.0, 0.01))
    idx = None
    if kind == 'sparse':
        g = np.random.default_rng(41)
        idx = np.stack([np.sort(g.choice(rows, k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
    override = 0 if kind == 'window' else -1

    def attend(stores, app):
        ek, ev, wk, wv = stores
        kw = dict(append_k=bf16_dev(raw_k), append_v=bf16_dev(raw_v)) if app else {}
        if kind == 'sparse':
            return v4.sparse_window_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'], dev(idx), **kw)
        return v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, m, wk, wv, c['W'], n_entries_override=override, **kw)

    print(f'attn fused append case {case} ({kind}, t={pos})', flush=True)
    sa = _stores(c)
    for b in range(B):
        v4.csa_compress(torch.zeros(1, 1, device='cuda'), torch.zeros(1, device='cuda'), int(q_pos[b, 0]),
                        bf16_dev(raw_k[b:b + 1]), bf16_dev(raw_v[b:b + 1]), _batch_view(sa[2], b),
                        _batch_view(sa[3], b))
    oa = attend(sa, False)
    sb = _stores(c)
    ob = attend(sb, True)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob), 'fused and separate append give different outputs'
    for x, y, n in ((sa[2], sb[2], 'win_k'), (sa[3], sb[3], 'win_v')):
        for pl in ('nope', 'rope', 'scale'):
            assert torch.equal(getattr(x, pl), getattr(y, pl)), f'{n}.{pl} differs'
    # the appended row against the oracle's m = 1 compression, and the output
    # against the oracle over the window that now holds it
    ob = ob.float().cpu().numpy()
    gk, gv = host_kv(sb[2]), host_kv(sb[3])
    for b in range(B):
        t = int(q_pos[b, 0])
        slot = t % ring if ring else t
        k32, v32, _ = OC.compress(raw_k[b:b + 1], raw_v[b:b + 1], np.zeros((1, 1), np.float32),
                                  np.zeros(1, np.float32), t)
        for name, x32, g in (('k', k32, gk), ('v', v32, gv)):
            codes, rope_bits, scale = F.kv_quantize(x32)
            assert np.array_equal(g['scale'][b:b + 1, slot:slot + 1], scale), f'{name}: scale b{b}'
            assert np.array_equal(g['rope'][b:b + 1, slot:slot + 1], rope_bits), f'{name}: rope b{b}'
            assert_codes_e4m3(g['nope'][b:b + 1, slot:slot + 1], codes, (x32[..., :128] / scale).astype(np.float32),
                              name)
        row = {n: {pl: a[b:b + 1, slot:slot + 1] for pl, a in g.items()} for n, g in (('wk', gk), ('wv', gv))}
        c['dec']['wk'][b, t - c['first']] = OC.decode_kv(row['wk'])[0, 0]
        c['dec']['wv'][b, t - c['first']] = OC.decode_kv(row['wv'])[0, 0]
        if kind == 'sparse':
            ids = idx[b, 0]
        else:
            ids = np.arange(0 if kind == 'window' else min((t + 1) // m, rows))
        ro, _ = _oracle_attn(c, b, 0, ids)
        assert_close_rms(ob[b, 0], ro, TOL_BF16, f'o b{b}')


# ---------------------------------------------------------- end to end ----

def test_c0_fp32_layer_end_to_end():
    """The fp32 CSA workload (4,096 tokens, decode of the last 16): compress, index, attend on the GPU."""
    cfg, x = synth.c0(0)
    T, D, m, k, W = cfg['T'], cfg['D'], cfg['m'], cfg['k'], cfg['W']
    N = T // m
    ks, vs = v4.KVStore.empty(1, N, D, v4.KV_F32), v4.KVStore.empty(1, N, D, v4.KV_F32)
    iks = v4.IKStore.empty(1, N, cfg['d_I'], v4.IK_F32)
    ring = 256    # holds the windows of all 16 queries (positions 3953 .. 4095)
    wk, wv = v4.KVStore.empty(1, ring, D, v4.KV_F32, ring), v4.KVStore.empty(1, ring, D, v4.KV_F32, ring)
    rk, rv, gate = dev(x['raw_k']), dev(x['raw_v']), dev(x['gate'])
    v4.csa_compress(gate, dev(x['pos_bias']), 0, rk, rv, ks, vs, dev(x['raw_ik']), iks)
    v4.csa_compress(gate, torch.zeros(1, device='cuda'), 0, rk, rv, wk, wv)
    q_pos = dev(x['q_pos'])
    idx = v4.lightning_index_topk(q_pos, dev(x['iq']), dev(x['w']), iks, k, m)
    o = v4.sparse_window_attn(dev(x['q']), q_pos, ks, vs, m, wk, wv, W, idx)
    torch.cuda.synchronize()
    idx, o = idx.cpu().numpy(), o.cpu().numpy()
    caches = OM.build_caches(x['raw_k'], x['raw_v'], x['gate'], x['pos_bias'], 'f32', raw_ik=x['raw_ik'], ik_fmt='f32')
    for i in range(cfg['Tq']):
        t = int(x['q_pos'][0, i])
        ro, _, sel, scores = OM.csa_query(x['q'][0, i], t, x['iq'][0, i], x['w'][0, i], caches['dik'][0],
                                          caches['dk'][0], caches['dv'][0], caches['dwk'][0], caches['dwv'][0], m, k, W)
        assert_topk(idx[0, i], scores, OI.n_visible(t, m, N), k, f'q{i}')
        if np.array_equal(np.sort(idx[0, i]), np.sort(sel)):
            assert_close_rms(o[0, i], ro, TOL_F32, f'o q{i}')
        else:   # a tie-band swap: check the GPU attention on the oracle's selection instead
            o2 = v4.sparse_window_attn(dev(x['q'][:, i:i + 1]), q_pos[:, i:i + 1], ks, vs, m, wk, wv, W,
                                       dev(sel[None, None]))
            assert_close_rms(o2.cpu().numpy()[0, 0], ro, TOL_F32, f'o q{i} (oracle selection)')


def test_empty_inputs():
    """Calls with nothing to do: compression of zero tokens leaves the stores as they
    were; an index call whose queries see no entry (t = -1, 0, 2 with m = 4) returns only
    padding; attention for a query with an empty key list (t = -1) gives o = 0 and
    lse = -inf, next to a query at t = 0 (window row 0 only) checked against the oracle."""
    B, D, m = 1, 192, 4
    ks, vs = v4.KVStore.empty(B, 8, D), v4.KVStore.empty(B, 8, D)
    iks = v4.IKStore.empty(B, 8, 128)
    for t in (ks.nope, vs.nope, iks.e2m1, iks.e8m0):
        t.fill_(0xAB)
    before = [t.clone() for t in (ks.nope, ks.rope, ks.scale, vs.nope, iks.e2m1, iks.e8m0)]
    g = torch.zeros(B, 8, device='cuda')
    raw = torch.ones(B, 8, D, dtype=torch.bfloat16, device='cuda')
    u = torch.ones(B, 8, 128, dtype=torch.bfloat16, device='cuda')
    print('empty compress', flush=True)
    v4.csa_compress(g[:, :0], torch.zeros(m, device='cuda'), 0, raw[:, :0], raw[:, :0], ks, vs, u[:, :0], iks)
    torch.cuda.synchronize()
    after = (ks.nope, ks.rope, ks.scale, vs.nope, iks.e2m1, iks.e8m0)
    assert all(torch.equal(a, b) for a, b in zip(before, after))

    q_pos = np.array([[-1, 0, 2]], np.int64)
    c = _index_case_mx(51, 1, 100, q_pos, 16)
    print('index with no visible entries', flush=True)
    idx, score = _run_index(c)
    assert np.all(idx == -1) and np.all(score == 0)

    q_pos = np.array([[-1, 0]], np.int64)
    a = _attn_case(52, 1, 2, 64, D, 50, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(a)
    ids = np.full((1, 2, 8), -1, np.int32)
    lse = torch.zeros(1, 2, 64, dtype=torch.float32, device='cuda')
    print('attention over empty key lists', flush=True)
    for name, o in (('sparse', v4.sparse_window_attn(_qdev(a), dev(q_pos), ek, ev, m, wk, wv, a['W'], dev(ids),
                                                      lse=lse)),
                    ('dense', v4.hca_attn(_qdev(a), dev(q_pos), ek, ev, m, wk, wv, a['W'], lse=lse))):
        torch.cuda.synchronize()
        o, l = o.float().cpu().numpy(), lse.cpu().numpy()
        assert np.all(o[0, 0] == 0) and np.all(np.isneginf(l[0, 0])), name
        ro, rl = _oracle_attn(a, 0, 1, np.arange(0))
        assert_close_rms(o[0, 1], ro, TOL_BF16, f'{name} t=0')
        assert np.allclose(l[0, 1], rl, atol=2e-2), name


def test_attn_bf16_output():
    """bfloat16 output: the kernel's error plus the output's own rounding (2^-8 relative)."""
    B, Tq, rows, H, D = 1, 2, 600, 64, 192
    q_pos = np.array([[2399, 1000]], np.int64)
    c = _attn_case(15, B, Tq, H, D, rows, q_pos, 'fp8')
    ek, ev, wk, wv = _stores(c)
    o = torch.empty(B, Tq, H, D, dtype=torch.bfloat16, device='cuda')
    v4.hca_attn(_qdev(c), dev(q_pos), ek, ev, 4, wk, wv, c['W'], o=o)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    for i in range(Tq):
        t = int(q_pos[0, i])
        ro, _ = _oracle_attn(c, 0, i, np.arange(min((t + 1) // 4, rows)))
        rms = np.sqrt(np.mean(ro ** 2))
        assert np.all(np.abs(o[0, i] - ro) <= TOL_BF16 * rms + 2.0 ** -8 * np.abs(ro))
