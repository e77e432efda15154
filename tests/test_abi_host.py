"""Host-side checks of the C ABI library (no GPU needed).

The library loads and exports every symbol include/v4attn.h declares, and
every malformed call is rejected with its status code before anything is
enqueued. Only invalid calls are made here: validation runs before any HIP
call, so no device is touched.
"""

import ctypes
import os
import re

import pytest

from long_context_attention_compress_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7f0000000000      # never dereferenced: every call below fails validation first


def _declared():
    src = open(os.path.join(ROOT, 'include', 'v4attn.h')).read()
    src = re.sub(r'/\*.*?\*/', '', src, flags=re.S)
    return set(re.findall(r'\b([a-z_0-9]+)\s*\([^;{]*\)\s*;', src)) - {'if', 'sizeof'}


def test_exports_every_declared_symbol():
    lib = _abi.load()
    names = _declared()
    assert {'csa_compress', 'lightning_index_topk', 'sparse_window_attn', 'hca_attn'} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert set(_abi.EXPORTS) == names


def test_strerror_and_version():
    lib = _abi.load()
    assert lib.v4a_strerror(0) == b'ok'
    assert lib.v4a_strerror(-5).startswith(b'workspace')
    assert b'gfx950' in lib.v4a_version()


def _plane(ptr=FAKE, rs=256, bs=256 * 4096):
    return _abi.Plane(ptr, rs, bs)


def _kv(fmt=_abi.KV_E4M3_BF16, dim=192, rows=4096, ring=0):
    s = _abi.KvStoreC()
    s.fmt, s.dim, s.rows, s.ring = fmt, dim, rows, ring
    if fmt == _abi.KV_F32:
        s.f32 = _plane(rs=4 * dim)
    else:
        s.nope, s.rope, s.scale = _plane(rs=128), _plane(rs=128), _plane(rs=4)
    return s


def _ik(fmt=_abi.IK_MXFP4, dim=128, rows=4096):
    s = _abi.IkStoreC()
    s.fmt, s.dim, s.rows = fmt, dim, rows
    s.e2m1, s.e8m0 = _plane(rs=64), _plane(rs=4)
    return s


def _status(fn, *args):
    lib = _abi.load()
    r = getattr(lib, fn)(*args)
    return r, lib.v4a_last_error().decode()


def test_compress_rejections():
    k, v, ik = _kv(), _kv(), _ik()

    def args(**kw):
        a = _abi.CompressArgs()
        a.B, a.t_new, a.pos0, a.m, a.act_fmt, a.rope_base = 2, 16, 0, 4, _abi.ACT_BF16, 1e4
        a.raw_k = a.raw_v = a.gate = a.pos_bias = a.raw_ik = FAKE
        a.k_out, a.v_out, a.ik_out = ctypes.pointer(k), ctypes.pointer(v), ctypes.pointer(ik)
        for n, val in kw.items():
            setattr(a, n, val)
        return ctypes.byref(a)

    cases = [
        (dict(m=0), _abi.V4A_EINVAL), (dict(m=2000), _abi.V4A_EINVAL), (dict(pos0=2), _abi.V4A_EINVAL),
        (dict(t_new=6), _abi.V4A_EINVAL), (dict(gate=None), _abi.V4A_ENULL), (dict(act_fmt=7), _abi.V4A_EFORMAT),
        (dict(raw_ik=None), _abi.V4A_ENULL), (dict(pos0=4096 * 4), _abi.V4A_EINVAL), (dict(raw_k=FAKE + 1), _abi.V4A_EALIGN),
        (dict(raw_v=FAKE + 2), _abi.V4A_EALIGN), (dict(raw_ik=FAKE + 2), _abi.V4A_EALIGN),
        (dict(t_new=4 * ((1 << 21) + 1)), _abi.V4A_EINVAL),
        (dict(k_out=None, v_out=None, ik_out=None, raw_ik=None), _abi.V4A_EINVAL), (dict(B=70000), _abi.V4A_EINVAL),
    ]
    for kw, want in cases:
        r, msg = _status('csa_compress', args(**kw), None)
        assert r == want, (kw, r, msg)
    # zero tokens: a no-op once the sizes are valid, whatever the pointers
    r, msg = _status('csa_compress', args(t_new=0, gate=None, raw_k=None, raw_v=None, raw_ik=None), None)
    assert r == _abi.V4A_OK, msg
    r, _ = _status('csa_compress', args(t_new=0, m=0), None)
    assert r == _abi.V4A_EINVAL
    bad_dim = _kv(dim=128)
    r, _ = _status('csa_compress', args(k_out=ctypes.pointer(bad_dim), v_out=ctypes.pointer(bad_dim)), None)
    assert r == _abi.V4A_EFORMAT
    bad_align = _kv()
    bad_align.nope = _plane(ptr=FAKE + 8)
    r, _ = _status('csa_compress', args(k_out=ctypes.pointer(bad_align)), None)
    assert r == _abi.V4A_EALIGN


def test_index_rejections():
    keys = _ik()

    def args(**kw):
        a = _abi.IndexArgs()
        a.B, a.Tq, a.H_I, a.k, a.m = 2, 1, 64, 512, 4
        a.q_pos = a.iq = a.iq_scale = a.w = a.out_idx = FAKE
        a.keys = ctypes.pointer(keys)
        for n, val in kw.items():
            setattr(a, n, val)
        return a

    lib = _abi.load()
    assert lib.lightning_index_topk_workspace(ctypes.byref(args())) > 0
    assert lib.lightning_index_topk_workspace(ctypes.byref(args(k=0))) == 0
    cases = [(dict(k=0), _abi.V4A_EINVAL), (dict(k=5000), _abi.V4A_EINVAL), (dict(H_I=20), _abi.V4A_EFORMAT),
             (dict(iq_scale=None), _abi.V4A_ENULL), (dict(q_pos=None), _abi.V4A_ENULL),
             (dict(iq=FAKE + 4), _abi.V4A_EALIGN), (dict(m=0), _abi.V4A_EINVAL)]
    for kw, want in cases:
        r, msg = _status('lightning_index_topk', ctypes.byref(args(**kw)), FAKE, 1 << 30, None)
        assert r == want, (kw, r, msg)
    # missing / short workspace
    r, _ = _status('lightning_index_topk', ctypes.byref(args()), None, 0, None)
    assert r == _abi.V4A_EWORKSPACE
    r, _ = _status('lightning_index_topk', ctypes.byref(args()), FAKE, 16, None)
    assert r == _abi.V4A_EWORKSPACE
    bad = _ik(dim=64)
    r, _ = _status('lightning_index_topk', ctypes.byref(args(keys=ctypes.pointer(bad))), FAKE, 1 << 30, None)
    assert r == _abi.V4A_EFORMAT


def test_attention_rejections():
    ek, ev, wk, wv = _kv(), _kv(), _kv(ring=128, rows=128), _kv(ring=128, rows=128)

    def args(**kw):
        a = _abi.AttnArgs()
        a.B, a.Tq, a.H_q, a.dim = 4, 1, 64, 192
        a.q_pos = a.q = a.o = FAKE
        a.q_fmt = a.o_fmt = _abi.ACT_BF16
        a.ent_k, a.ent_v, a.win_k, a.win_v = (ctypes.pointer(s) for s in (ek, ev, wk, wv))
        a.m, a.W, a.sm_scale, a.rope_base = 4, 128, 0.0, 1e4
        for n, val in kw.items():
            setattr(a, n, val)
        return ctypes.byref(a)

    lib = _abi.load()
    assert lib.hca_attn_workspace(args(), -1) > 0
    f32 = _kv(fmt=_abi.KV_F32, dim=192)
    cases = [(dict(H_q=24), _abi.V4A_EFORMAT), (dict(q_fmt=_abi.ACT_F32), _abi.V4A_EFORMAT),
             (dict(W=-1), _abi.V4A_EINVAL), (dict(q=None), _abi.V4A_ENULL), (dict(o=FAKE + 2), _abi.V4A_EALIGN),
             (dict(ent_v=None), _abi.V4A_ENULL), (dict(sm_scale=float('nan')), _abi.V4A_EINVAL),
             (dict(ent_k=ctypes.pointer(f32)), _abi.V4A_EFORMAT), (dict(dim=128), _abi.V4A_EFORMAT)]
    for kw, want in cases:
        r, msg = _status('hca_attn', args(**kw), -1, FAKE, 1 << 30, None)
        assert r == want, (kw, r, msg)
    r, _ = _status('hca_attn', args(), -1, None, 0, None)
    assert r == _abi.V4A_EWORKSPACE
    r, _ = _status('sparse_window_attn', args(), None, 1024, FAKE, 1 << 30, None)
    assert r == _abi.V4A_ENULL
    r, _ = _status('sparse_window_attn', args(), FAKE, 0, FAKE, 1 << 30, None)
    assert r == _abi.V4A_EINVAL
    ring_ent = _kv(ring=64)
    r, _ = _status('hca_attn', args(ent_k=ctypes.pointer(ring_ent)), -1, FAKE, 1 << 30, None)
    assert r == _abi.V4A_EINVAL
    # fused window append: both rows or neither, one query token per sequence,
    # a window, 4-byte alignment, FP8 stores only
    app = dict(append_k=FAKE, append_v=FAKE)
    f32s = [ctypes.pointer(_kv(fmt=_abi.KV_F32, dim=128, ring=r_, rows=128 if r_ else 4096)) for r_ in (0, 0, 128, 128)]
    f32_args = dict(ent_k=f32s[0], ent_v=f32s[1], win_k=f32s[2], win_v=f32s[3], dim=128, H_q=16,
                    q_fmt=_abi.ACT_F32, o_fmt=_abi.ACT_F32)
    assert lib.hca_attn_workspace(args(**f32_args), -1) > 0   # valid without the append
    app_cases = [(dict(append_k=FAKE), _abi.V4A_ENULL), (dict(append_v=FAKE), _abi.V4A_ENULL),
                 (dict(app, Tq=2), _abi.V4A_EINVAL), (dict(app, W=0), _abi.V4A_EINVAL),
                 (dict(app, append_v=FAKE + 2), _abi.V4A_EALIGN), (dict(app, **f32_args), _abi.V4A_EFORMAT)]
    for kw, want in app_cases:
        r, msg = _status('hca_attn', args(**kw), -1, FAKE, 1 << 30, None)
        assert r == want, (kw, r, msg)
    r, msg = _status('sparse_window_attn', args(**dict(app, Tq=3)), FAKE, 1024, FAKE, 1 << 30, None)
    assert r == _abi.V4A_EINVAL and 'Tq' in msg, (r, msg)
    assert lib.hca_attn_workspace(args(**app), -1) > 0


def test_attention_key_list_and_ring_limits():
    """A key list longer than the splits can resolve, a window ring shorter than the
    window and a store of 2^30 rows or more are rejected before any launch (and their
    workspace size is 0)."""
    lib = _abi.load()
    big = 1024 * 2048   # splits per query x keys a split resolves

    def args(ek_rows=4096, ring=128, W=128):
        a = _abi.AttnArgs()
        ek, ev = _kv(rows=ek_rows), _kv(rows=ek_rows)
        wk, wv = _kv(ring=ring, rows=max(ring, 128)), _kv(ring=ring, rows=max(ring, 128))
        a._keep = (ek, ev, wk, wv)
        a.B, a.Tq, a.H_q, a.dim = 1, 1, 64, 192
        a.q_pos = a.q = a.o = FAKE
        a.q_fmt = a.o_fmt = _abi.ACT_BF16
        a.ent_k, a.ent_v, a.win_k, a.win_v = (ctypes.pointer(s) for s in (ek, ev, wk, wv))
        a.m, a.W, a.sm_scale, a.rope_base = 1, W, 0.0, 1e4
        return a

    ok = args(ek_rows=big - 128)
    assert lib.hca_attn_workspace(ctypes.byref(ok), -1) > 0
    over = args(ek_rows=big - 127)
    assert lib.hca_attn_workspace(ctypes.byref(over), -1) == 0
    r, msg = _status('hca_attn', ctypes.byref(over), -1, FAKE, 1 << 40, None)
    assert r == _abi.V4A_EINVAL and 'key list' in msg, (r, msg)
    # capped by the override: accepted again
    assert lib.hca_attn_workspace(ctypes.byref(over), 1000) > 0
    # sparse: the list is k long
    sp = args()
    assert lib.sparse_window_attn_workspace(ctypes.byref(sp), 65536) > 0
    r, _ = _status('sparse_window_attn', ctypes.byref(sp), FAKE, 65537, FAKE, 1 << 40, None)
    assert r == _abi.V4A_EINVAL
    # window ring: at least W slots
    short = args(ring=100, W=128)
    assert lib.hca_attn_workspace(ctypes.byref(short), -1) == 0
    r, msg = _status('hca_attn', ctypes.byref(short), -1, FAKE, 1 << 30, None)
    assert r == _abi.V4A_EINVAL and 'ring' in msg, (r, msg)
    assert lib.hca_attn_workspace(ctypes.byref(args(ring=128, W=128)), -1) > 0
    assert lib.hca_attn_workspace(ctypes.byref(args(ring=100, W=100)), -1) > 0
    # store rows are addressed by 30-bit codes: 2^30 rows or more are rejected
    huge = args(ek_rows=1 << 30)
    assert lib.hca_attn_workspace(ctypes.byref(huge), 1000) == 0
    r, msg = _status('hca_attn', ctypes.byref(huge), 1000, FAKE, 1 << 40, None)
    assert r == _abi.V4A_EINVAL and '2^30' in msg, (r, msg)
    assert lib.hca_attn_workspace(ctypes.byref(args(ek_rows=(1 << 30) - 1)), 1000) > 0


def test_index_noalloc_rejections():
    """The workspace-free indexer call validates like lightning_index_topk and rejects a call
    whose scratch would exceed the static array, before touching any device."""
    keys = _ik(rows=262144)

    def args(**kw):
        a = _abi.IndexArgs()
        a.B, a.Tq, a.H_I, a.k, a.m = 4, 1, 64, 1024, 4
        a.q_pos = a.iq = a.iq_scale = a.w = a.out_idx = FAKE
        a.keys = ctypes.pointer(keys)
        for n, val in kw.items():
            setattr(a, n, val)
        return a

    lib = _abi.load()
    need = lib.lightning_index_topk_workspace(ctypes.byref(args()))
    assert 0 < need <= _abi.NOALLOC_SCRATCH_BYTES
    for kw, want in [(dict(k=0), _abi.V4A_EINVAL), (dict(q_pos=None), _abi.V4A_ENULL),
                     (dict(iq=FAKE + 4), _abi.V4A_EALIGN), (dict(H_I=20), _abi.V4A_EFORMAT)]:
        r, msg = _status('lightning_index_topk_noalloc', ctypes.byref(args(**kw)), None)
        assert r == want, (kw, r, msg)
    big = args(Tq=1000)
    assert lib.lightning_index_topk_workspace(ctypes.byref(big)) > _abi.NOALLOC_SCRATCH_BYTES
    r, msg = _status('lightning_index_topk_noalloc', ctypes.byref(big), None)
    assert r == _abi.V4A_EWORKSPACE and 'static scratch' in msg, (r, msg)


def test_compress_block_mode_rejections():
    """Block mode (device positions) needs pos0 == 0, a raw ring of at least m rows and an
    8-byte aligned position array; a linear store's rows are checked on the device then."""
    k, v = _kv(rows=16), _kv(rows=16)

    def args(**kw):
        a = _abi.CompressArgs()
        a.B, a.t_new, a.pos0, a.m, a.act_fmt, a.rope_base = 2, 8, 0, 4, _abi.ACT_BF16, 1e4
        a.raw_k = a.raw_v = a.gate = a.pos_bias = FAKE
        a.k_out, a.v_out = ctypes.pointer(k), ctypes.pointer(v)
        a.block_end = FAKE
        for n, val in kw.items():
            setattr(a, n, val)
        return ctypes.byref(a)

    for kw, want in [(dict(pos0=4), _abi.V4A_EINVAL), (dict(t_new=0), _abi.V4A_EINVAL), (dict(block_end=FAKE + 4),
                     _abi.V4A_EALIGN)]:
        r, msg = _status('csa_compress', args(**kw), None)
        assert r == want, (kw, r, msg)
    a = _abi.CompressArgs()
    a.B, a.t_new, a.pos0, a.m, a.act_fmt, a.rope_base = 2, 4, 0, 8, _abi.ACT_BF16, 1e4
    a.raw_k = a.raw_v = a.gate = a.pos_bias = FAKE
    a.k_out, a.v_out = ctypes.pointer(k), ctypes.pointer(v)
    a.block_end = FAKE
    r, msg = _status('csa_compress', ctypes.byref(a), None)
    assert r == _abi.V4A_EINVAL, (r, msg)      # t_new = 4 is not a multiple of m = 8
