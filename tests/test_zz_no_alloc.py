"""The workspace-free indexer call (lightning_index_topk_noalloc) against lightning_index_topk.

Through the C ABI: two calls in a row, the second with a smaller input, each
compared bitwise (selected ids and scores) with lightning_index_topk given its
own workspace on the same inputs. The first case also goes against the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import long_context_attention_compress_amd as v4
import synth
from long_context_attention_compress_amd import _abi
from oracle import formats as F
from oracle import indexer as OI
from tests.helpers import assert_topk, dev

pytestmark = pytest.mark.gpu


def _case(seed, B, rows, q_pos, k):
    H, dI = 64, 128
    keys = synth.normal(seed, 'na/ik', (B, rows, dI))
    iq = synth.normal(seed, 'na/iq', (B, q_pos.shape[1], H, dI), outlier_frac=0.01)
    w = synth.uniform(seed, 'na/w', (B, q_pos.shape[1], H))
    packed, sc = F.mxfp4_quantize(keys)
    ip, isc = F.mxfp4_quantize(iq)
    return dict(packed=packed, sc=sc, ip=ip, isc=isc, w=w, q_pos=q_pos, k=k)


def _args(c, store, idx, score, t):
    B, Tq = c['q_pos'].shape
    a = _abi.IndexArgs()
    a.B, a.Tq, a.H_I, a.k, a.m = B, Tq, 64, c['k'], 4
    a.q_pos, a.iq, a.iq_scale, a.w = (t[n].data_ptr() for n in ('q_pos', 'iq', 'isc', 'w'))
    a.keys = store.c()
    a.out_idx, a.out_score = idx.data_ptr(), score.data_ptr()
    return a


def _run_both(c):
    B, Tq = c['q_pos'].shape
    store = v4.IKStore(v4.IK_MXFP4, 128, e2m1=dev(c['packed']), e8m0=dev(c['sc']))
    t = dict(q_pos=dev(c['q_pos']), iq=dev(c['ip']), isc=dev(c['isc']), w=dev(c['w']))
    lib = _abi.load()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    out = []
    for noalloc in (False, True):
        idx = torch.full((B, Tq, c['k']), -7, dtype=torch.int32, device='cuda')
        score = torch.full((B, Tq, c['k']), 7.0, dtype=torch.float32, device='cuda')
        a = _args(c, store, idx, score, t)
        if noalloc:
            r = lib.lightning_index_topk_noalloc(ctypes.byref(a), stream)
        else:
            n = lib.lightning_index_topk_workspace(ctypes.byref(a))
            ws = torch.empty(n, dtype=torch.uint8, device='cuda')
            assert lib.v4a_workspace_init(ws.data_ptr(), n, stream) == 0
            r = lib.lightning_index_topk(ctypes.byref(a), ws.data_ptr(), n, stream)
        assert r == 0, lib.v4a_last_error().decode()
        torch.cuda.synchronize()
        out.append((idx.cpu().numpy(), score.cpu().numpy()))
    (i0, s0), (i1, s1) = out
    assert np.array_equal(i0, i1), 'selected ids differ between the two entry points'
    assert np.array_equal(s0.view(np.uint32), s1.view(np.uint32)), 'scores differ between the two entry points'
    return i1


def test_noalloc_matches_workspace_call_twice():
    q_pos = np.array([[20000 * 4 - 1, 12345, 7], [5000, 20000 * 4 - 1, -1]], np.int64)
    c = _case(51, 2, 20000, q_pos, 512)
    print('noalloc call 1: B=2 Tq=3 rows=20000 k=512', flush=True)
    idx = _run_both(c)
    dk, diq = F.mxfp4_dequantize(c['packed'], c['sc']), F.mxfp4_dequantize(c['ip'], c['isc'])
    for b in range(2):
        for i in range(3):
            t = int(q_pos[b, i])
            n_vis = OI.n_visible(t, 4, 20000) if t >= 0 else 0
            assert_topk(idx[b, i], OI.index_scores(diq[b, i], c['w'][b, i], dk[b, :n_vis]), n_vis, 512, f'b{b} i{i}')
    c2 = _case(52, 1, 3000, np.array([[3000 * 4 - 1]], np.int64), 256)
    print('noalloc call 2 (smaller): B=1 Tq=1 rows=3000 k=256', flush=True)
    _run_both(c2)
