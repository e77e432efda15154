"""Python binding of libv4attn: hybrid compressed attention (CSA / HCA) for MI355X.

Argument marshalling only: every step of the path (compression, indexer
scoring and top-k, sparse and dense window attention) runs in the HIP kernels
of libv4attn.so. torch supplies device memory and the current stream.

Entry points (same names as the C ABI in include/v4attn.h):
    csa_compress, lightning_index_topk, sparse_window_attn, hca_attn
Stores:
    KVStore  key/value cache (float32, or E4M3 no-RoPE dims + BF16 RoPE dims)
    IKStore  indexer-key cache (float32, or MXFP4)
"""

import ctypes

import torch

from . import _abi
from ._abi import (ACT_BF16, ACT_F32, IK_F32, IK_MXFP4, KV_E4M3_BF16, KV_F32, POOL_BLOCK, POOL_CHANNEL_GATE,
                   POOL_OVERLAP, POOL_ROPE_AFTER)

__all__ = ['KVStore', 'IKStore', 'Workspace', 'V4AError', 'Call', 'csa_compress', 'lightning_index_topk',
           'lightning_index_topk_noalloc', 'sparse_window_attn', 'hca_attn', 'lib', 'ROPE_DIM']

ROPE_DIM = 64


class V4AError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f'v4attn status {status}: {msg}')
        self.status = status


def lib():
    return _abi.load()


def _check(status):
    if status != 0:
        raise V4AError(status, lib().v4a_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _plane(t, row_dim=1):
    """Plane descriptor of a [B, rows, ...] tensor (strides in bytes)."""
    if t is None:
        return _abi.Plane(None, 0, 0)
    es = t.element_size()
    return _abi.Plane(t.data_ptr(), t.stride(row_dim) * es, t.stride(0) * es)


class KVStore:
    """A key or value store of B x rows rows of `dim` values (the last 64 are RoPE dims).

    fmt KV_F32:       f32   [B, rows, dim] float32
    fmt KV_E4M3_BF16: nope  [B, rows, dim-64] uint8 (OCP E4M3 codes),
                      rope  [B, rows, 64] int16 (bfloat16 bits),
                      scale [B, rows, (dim-64)//128] float32
    ring > 0 maps position/entry n to row n % ring.
    """

    def __init__(self, fmt, dim, ring=0, f32=None, nope=None, rope=None, scale=None):
        self.fmt, self.dim, self.ring = fmt, dim, ring
        self.f32, self.nope, self.rope, self.scale = f32, nope, rope, scale
        ref = f32 if fmt == KV_F32 else nope
        self.B, self.rows = ref.shape[0], ref.shape[1]
        self._c = _abi.KvStoreC(fmt, dim, self.rows, ring, _plane(f32), _plane(nope), _plane(rope), _plane(scale))

    @classmethod
    def empty(cls, B, rows, dim, fmt=KV_E4M3_BF16, ring=0, device='cuda'):
        if fmt == KV_F32:
            return cls(fmt, dim, ring, f32=torch.zeros(B, rows, dim, dtype=torch.float32, device=device))
        dn = dim - ROPE_DIM
        return cls(fmt, dim, ring,
                   nope=torch.zeros(B, rows, dn, dtype=torch.uint8, device=device),
                   rope=torch.zeros(B, rows, ROPE_DIM, dtype=torch.int16, device=device),
                   scale=torch.zeros(B, rows, dn // 128, dtype=torch.float32, device=device))

    def c(self):
        return ctypes.pointer(self._c)


class IKStore:
    """Indexer keys: fmt IK_F32 -> f32 [B, rows, dim]; IK_MXFP4 -> e2m1 [B, rows, dim/2] uint8
    (element 2i in the low nibble of byte i) and e8m0 [B, rows, dim/32] uint8."""

    def __init__(self, fmt, dim, f32=None, e2m1=None, e8m0=None):
        self.fmt, self.dim = fmt, dim
        self.f32, self.e2m1, self.e8m0 = f32, e2m1, e8m0
        ref = f32 if fmt == IK_F32 else e2m1
        self.B, self.rows = ref.shape[0], ref.shape[1]
        self._c = _abi.IkStoreC(fmt, dim, self.rows, _plane(f32), _plane(e2m1), _plane(e8m0))

    @classmethod
    def empty(cls, B, rows, dim, fmt=IK_MXFP4, device='cuda'):
        if fmt == IK_F32:
            return cls(fmt, dim, f32=torch.zeros(B, rows, dim, dtype=torch.float32, device=device))
        return cls(fmt, dim, e2m1=torch.zeros(B, rows, dim // 2, dtype=torch.uint8, device=device),
                   e8m0=torch.zeros(B, rows, dim // 32, dtype=torch.uint8, device=device))

    def c(self):
        return ctypes.pointer(self._c)


class Workspace:
    """Device scratch for the calls that need one, initialised once (v4a_workspace_init).

    Calls that may overlap in time on different streams need different Workspace objects.
    """

    def __init__(self, device='cuda'):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes, stream=None):
        if nbytes == 0:
            return None, 0
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 4096), dtype=torch.uint8, device=self.device)
            _check(lib().v4a_workspace_init(_ptr(self.buf), self.buf.numel(), _stream(stream)))
        return _ptr(self.buf), self.buf.numel()


_default_ws = {}


def _workspace(ws, tensor, kind):
    if ws is not None:
        return ws
    key = (tensor.device, kind)
    if key not in _default_ws:
        _default_ws[key] = Workspace(tensor.device)
    return _default_ws[key]


def _act(t):
    if t.dtype == torch.float32:
        return ACT_F32
    if t.dtype == torch.bfloat16:
        return ACT_BF16
    raise TypeError(f'unsupported activation dtype {t.dtype}')


def _need(t, name, dtype=None):
    if t is None:
        raise ValueError(f'{name} is required')
    if not t.is_contiguous():
        raise ValueError(f'{name} must be contiguous')
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f'{name} must be {dtype}, got {t.dtype}')
    return t


class Call:
    """A prepared launch: the argument structs are built once; calling it only enqueues.

    It keeps references to every tensor, store and workspace buffer it points at.
    """

    def __init__(self, fn, args, keep):
        self.fn, self.args, self.keep = fn, args, keep

    def __call__(self):
        _check(self.fn(*self.args))


def _finish(fn, args, keep, prepare):
    call = Call(fn, args, keep)
    if prepare:
        return call
    call()
    return None


def csa_compress(gate, pos_bias, pos0, raw_k=None, raw_v=None, k_out=None, v_out=None,
                 raw_ik=None, ik_out=None, rope_base=10000.0, stream=None, prepare=False, block_end=None,
                 variant=POOL_BLOCK):
    """Pool blocks of m raw tokens into entries pos0/m ... of the stores.

    m = len(pos_bias) (POOL_BLOCK, POOL_ROPE_AFTER), len(pos_bias) / 2 (POOL_OVERLAP, whose raw
    inputs and gate start m positions before pos0), pos_bias.shape[0] (POOL_CHANNEL_GATE, gate
    [B, T, C] and pos_bias [m, C]).
    block_end [B] int64 (device): block mode, the one block ending at each position (when it
    completes a block), raw inputs being rings of gate.shape[1] rows indexed by position.
    With prepare=True nothing is launched; a Call that enqueues this operation is returned."""
    _need(gate, 'gate', torch.float32)
    _need(pos_bias, 'pos_bias', torch.float32)
    ref = raw_k if raw_k is not None else raw_ik
    B, T = gate.shape[:2]
    if variant == POOL_OVERLAP:
        m = pos_bias.numel() // 2
        if block_end is None:
            T -= m          # the first m rows are the block before pos0
    elif variant == POOL_CHANNEL_GATE:
        m = pos_bias.shape[0]
    else:
        m = pos_bias.numel()
    a = _abi.CompressArgs()
    a.B, a.t_new, a.pos0, a.m = B, T, int(pos0), m
    a.variant = variant
    a.act_fmt = _act(ref)
    a.rope_base = rope_base
    if raw_k is not None:
        _need(raw_k, 'raw_k')
        _need(raw_v, 'raw_v', raw_k.dtype)
        a.raw_k, a.raw_v = _ptr(raw_k), _ptr(raw_v)
        a.k_out, a.v_out = k_out.c(), v_out.c()
    if raw_ik is not None:
        _need(raw_ik, 'raw_ik', ref.dtype)
        a.raw_ik = _ptr(raw_ik)
        a.ik_out = ik_out.c()
    a.gate, a.pos_bias = _ptr(gate), _ptr(pos_bias)
    if block_end is not None:
        a.block_end = _ptr(_need(block_end, 'block_end', torch.int64))
    keep = (a, gate, pos_bias, raw_k, raw_v, k_out, v_out, raw_ik, ik_out, block_end)
    return _finish(lib().csa_compress, (ctypes.byref(a), _stream(stream)), keep, prepare)


def lightning_index_topk(q_pos, iq, w, keys, k, m, iq_scale=None, out_idx=None, out_score=None,
                         workspace=None, stream=None, prepare=False):
    """Top-k entry ids per query: q_pos [B, Tq] int64; iq [B, Tq, H_I, dim/2] uint8 (MXFP4)
    with iq_scale [B, Tq, H_I, dim/32] uint8, or [B, Tq, H_I, dim] float32; w [B, Tq, H_I]."""
    _need(q_pos, 'q_pos', torch.int64)
    _need(iq, 'iq')
    _need(w, 'w', torch.float32)
    B, Tq, H = w.shape
    if out_idx is None:
        out_idx = torch.empty(B, Tq, k, dtype=torch.int32, device=w.device)
    a = _abi.IndexArgs()
    a.B, a.Tq, a.H_I, a.k, a.m = B, Tq, H, k, m
    a.q_pos, a.iq, a.w = _ptr(q_pos), _ptr(iq), _ptr(w)
    a.iq_scale = _ptr(_need(iq_scale, 'iq_scale')) if iq_scale is not None else None
    a.keys = keys.c()
    a.out_idx = _ptr(_need(out_idx, 'out_idx', torch.int32))
    a.out_score = _ptr(out_score) if out_score is not None else None
    L = lib()
    nbytes = L.lightning_index_topk_workspace(ctypes.byref(a))
    ws = _workspace(workspace, w, 'index')
    ptr, size = ws.get(nbytes, stream)
    keep = (a, q_pos, iq, iq_scale, w, keys, out_idx, out_score, ws.buf)
    call = _finish(L.lightning_index_topk, (ctypes.byref(a), ptr, size, _stream(stream)), keep, prepare)
    return call if prepare else out_idx


def lightning_index_topk_noalloc(q_pos, iq, w, keys, k, m, iq_scale=None, out_idx=None, out_score=None,
                                 stream=None, prepare=False):
    """lightning_index_topk with the library's static per-GPU scratch instead of a workspace
    (the call itself allocates nothing; calls that overlap on one GPU race on the scratch)."""
    _need(q_pos, 'q_pos', torch.int64)
    _need(iq, 'iq')
    _need(w, 'w', torch.float32)
    B, Tq, H = w.shape
    if out_idx is None:
        out_idx = torch.empty(B, Tq, k, dtype=torch.int32, device=w.device)
    a = _abi.IndexArgs()
    a.B, a.Tq, a.H_I, a.k, a.m = B, Tq, H, k, m
    a.q_pos, a.iq, a.w = _ptr(q_pos), _ptr(iq), _ptr(w)
    a.iq_scale = _ptr(_need(iq_scale, 'iq_scale')) if iq_scale is not None else None
    a.keys = keys.c()
    a.out_idx = _ptr(_need(out_idx, 'out_idx', torch.int32))
    a.out_score = _ptr(out_score) if out_score is not None else None
    keep = (a, q_pos, iq, iq_scale, w, keys, out_idx, out_score)
    call = _finish(lib().lightning_index_topk_noalloc, (ctypes.byref(a), _stream(stream)), keep, prepare)
    return call if prepare else out_idx


def _attn_args(q, q_pos, ent_k, ent_v, m, win_k, win_v, W, sm_scale, rope_base, o, lse, append_k, append_v):
    _need(q, 'q')
    _need(q_pos, 'q_pos', torch.int64)
    B, Tq, H, D = q.shape
    if o is None:   # float32 output by default (bfloat16 output is available by passing o)
        o = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    a = _abi.AttnArgs()
    a.B, a.Tq, a.H_q, a.dim = B, Tq, H, D
    a.q_pos, a.q_fmt, a.q = _ptr(q_pos), _act(q), _ptr(q)
    if ent_k is not None:
        a.ent_k, a.ent_v = ent_k.c(), ent_v.c()
    a.m = m
    a.win_k, a.win_v, a.W = win_k.c(), win_v.c(), W
    a.sm_scale, a.rope_base = sm_scale, rope_base
    a.o_fmt, a.o = _act(_need(o, 'o')), _ptr(o)
    a.lse = _ptr(lse) if lse is not None else None
    if append_k is not None or append_v is not None:
        a.append_k = _ptr(_need(append_k, 'append_k', torch.bfloat16))
        a.append_v = _ptr(_need(append_v, 'append_v', torch.bfloat16))
    return a, o


def sparse_window_attn(q, q_pos, ent_k, ent_v, m, win_k, win_v, W, idx, sm_scale=0.0,
                       rope_base=10000.0, o=None, lse=None, workspace=None, stream=None, prepare=False,
                       append_k=None, append_v=None):
    """CSA attention over the entries idx [B, Tq, k] (int32, -1 padded) plus the window.

    append_k/append_v [B, 1, dim] bfloat16 (decode): the query tokens' raw rows, first
    written into the window stores at the query positions (fused window append)."""
    a, o = _attn_args(q, q_pos, ent_k, ent_v, m, win_k, win_v, W, sm_scale, rope_base, o, lse, append_k, append_v)
    _need(idx, 'idx', torch.int32)
    k = idx.shape[-1]
    L = lib()
    nbytes = L.sparse_window_attn_workspace(ctypes.byref(a), k)
    ws = _workspace(workspace, q, 'attn')
    ptr, size = ws.get(nbytes, stream)
    keep = (a, q, q_pos, ent_k, ent_v, win_k, win_v, idx, o, lse, append_k, append_v, ws.buf)
    call = _finish(L.sparse_window_attn, (ctypes.byref(a), _ptr(idx), k, ptr, size, _stream(stream)), keep, prepare)
    return call if prepare else o


def hca_attn(q, q_pos, ent_k, ent_v, m, win_k, win_v, W, n_entries_override=-1, sm_scale=0.0,
             rope_base=10000.0, o=None, lse=None, workspace=None, stream=None, prepare=False,
             append_k=None, append_v=None):
    """HCA attention over every visible entry plus the window (n_entries_override=0: window only).

    append_k/append_v: fused window append, as in sparse_window_attn."""
    a, o = _attn_args(q, q_pos, ent_k, ent_v, m, win_k, win_v, W, sm_scale, rope_base, o, lse, append_k, append_v)
    L = lib()
    nbytes = L.hca_attn_workspace(ctypes.byref(a), n_entries_override)
    ws = _workspace(workspace, q, 'attn')
    ptr, size = ws.get(nbytes, stream)
    keep = (a, q, q_pos, ent_k, ent_v, win_k, win_v, o, lse, append_k, append_v, ws.buf)
    call = _finish(L.hca_attn, (ctypes.byref(a), n_entries_override, ptr, size, _stream(stream)), keep, prepare)
    return call if prepare else o
