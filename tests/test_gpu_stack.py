"""Decode steps through a small attention stack, replayed from one captured HIP graph while
the position advances, against the oracle layer by layer.

[golem.de, "Chinas KI-Unabhängigkeit?: Bei Deepseek V4 haben kleine Änderungen große
Wirkung", section "Komprimierte Erinnerung für längere Kontexte"]: the first layers
attend over the window alone; [chaosnode.de, "DeepSeek-V4: 1 Million Token Context
endlich nutzbar", section "Hybrid Attention: CSA und HCA"]: CSA and HCA layers
alternate, CSA pooling blocks of 4 tokens and HCA blocks of 128.

The stack is window-only, CSA, HCA, CSA (B = 2, 1,020 tokens of context, then 16
decode steps at positions 1,020 .. 1,035). One step is captured once: for every layer
the block compression in block mode (it writes the entry of the block that the step's
token completes, at device positions), the indexer for CSA, and the attention with the
fused window append. Between replays the program writes the next token's inputs (its
raw rows into the layers' raw rings, queries, the position) eagerly, as a decode loop
would. CSA blocks complete at t = 1,023, 1,027, 1,031, 1,035 and the HCA block of 128
at t = 1,023, so their new entries are seen by the same step's queries. The first two
steps also run eagerly: replay and eager outputs are bitwise equal. Every step's output
of every layer is checked against the oracle's own compression of the raw history, and
the entries and window rows the graph wrote against the oracle's encoding.
"""

import numpy as np
import pytest
import torch

import long_context_attention_compress_amd as v4
import synth
from oracle import attention as OA
from oracle import compress as OC
from oracle import formats as F
from oracle import indexer as OI
from oracle import model as OM
from tests.helpers import TOL_BF16, assert_close_rms, assert_kv_rows, assert_topk, bf16_dev, dev, kv_planes

pytestmark = pytest.mark.gpu

B, D, H, HI, DI, K, W = 2, 192, 64, 64, 128, 64, 128
T0, S = 1020, 16
KINDS = ('win', 'csa', 'hca', 'csa')
M_OF = {'csa': 4, 'hca': 128, 'win': 128}


def _oracle_layer(kind, r):
    """The oracle's caches of one layer from its raw history: dequantized entries of every
    block complete by the last step, window rows of every position (row p = position p),
    and the float32 rows (for the cache-plane checks)."""
    TT = T0 + S
    m = M_OF[kind]
    out = {}
    if kind != 'win':
        nb = TT // m
        k32, v32, u32 = OC.compress(r['raw_k'][:, :nb * m], r['raw_v'][:, :nb * m], r['gate'][:, :nb * m],
                                    r['pos_bias'], 0, raw_ik=r['raw_ik'][:, :nb * m] if kind == 'csa' else None)
        out.update(k32=k32, v32=v32, dk=F.kv_dequantize(*F.kv_quantize(k32)), dv=F.kv_dequantize(*F.kv_quantize(v32)))
        if kind == 'csa':
            out['dik'] = F.mxfp4_dequantize(*F.mxfp4_quantize(u32))
    wk32, wv32, _ = OC.compress(r['raw_k'], r['raw_v'], np.zeros((B, TT), np.float32), np.zeros(1, np.float32), 0)
    out.update(wk32=wk32, wv32=wv32, dwk=F.kv_dequantize(*F.kv_quantize(wk32)),
               dwv=F.kv_dequantize(*F.kv_quantize(wv32)))
    return out


def test_stack_decode_steps_advance_against_oracle():
    TT = T0 + S
    raws = [synth.raw_tokens(700 + l, B, TT, D, M_OF[kind], DI if kind == 'csa' else 0, bf16=True,
                             prefix=f'stack/{l}') for l, kind in enumerate(KINDS)]
    qs = [synth.queries(710 + l, B, S, H, D, HI, DI, outlier_frac=0.01, prefix=f'stackq/{l}')
          for l in range(len(KINDS))]
    s = torch.cuda.Stream()
    pos = torch.zeros(B, 1, dtype=torch.int64, device='cuda')
    pos_b = pos.view(B)
    z1 = torch.zeros(1, device='cuda')
    wsi, wsa = v4.Workspace(), v4.Workspace()
    layers = []
    with torch.cuda.stream(s):
        for l, kind in enumerate(KINDS):
            r, q = raws[l], qs[l]
            m = M_OF[kind]
            L = dict(kind=kind, rk=bf16_dev(r['raw_k']), rv=bf16_dev(r['raw_v']), g=dev(r['gate']),
                     bias=dev(r['pos_bias']), q_all=bf16_dev(q['q']))
            L['q'] = torch.empty(B, 1, H, D, dtype=torch.bfloat16, device='cuda')
            L['ak'] = torch.empty(B, 1, D, dtype=torch.bfloat16, device='cuda')
            L['av'] = torch.empty(B, 1, D, dtype=torch.bfloat16, device='cuda')
            L['o'] = torch.zeros(B, 1, H, D, device='cuda')
            # window ring: positions T0 - W .. T0 - 1 (the step's own row comes from the fused append)
            L['wk'], L['wv'] = v4.KVStore.empty(B, W, D, ring=W), v4.KVStore.empty(B, W, D, ring=W)
            v4.csa_compress(torch.zeros(B, W, device='cuda'), z1, T0 - W, L['rk'][:, T0 - W:T0].contiguous(),
                            L['rv'][:, T0 - W:T0].contiguous(), L['wk'], L['wv'])
            calls = []
            if kind == 'win':
                calls.append(v4.hca_attn(L['q'], pos, None, None, m, L['wk'], L['wv'], W, n_entries_override=0,
                                         o=L['o'], workspace=wsa, prepare=True, append_k=L['ak'], append_v=L['av']))
            else:
                rows = TT // m + 1
                L['ek'], L['ev'] = v4.KVStore.empty(B, rows, D), v4.KVStore.empty(B, rows, D)
                L['ru'] = bf16_dev(r['raw_ik']) if kind == 'csa' else None
                L['ik'] = v4.IKStore.empty(B, rows, DI) if kind == 'csa' else None
                nb0 = T0 // m        # blocks complete before the first step
                v4.csa_compress(L['g'][:, :nb0 * m].contiguous(), L['bias'], 0, L['rk'][:, :nb0 * m].contiguous(),
                                L['rv'][:, :nb0 * m].contiguous(), L['ek'], L['ev'],
                                None if L['ru'] is None else L['ru'][:, :nb0 * m].contiguous(), L['ik'])
                # raw rings of the block compression: position p at row p % R (R = m);
                # the pending tokens of the open block are in place
                R = m
                L['R'] = R
                L['ring_k'] = torch.zeros(B, R, D, dtype=torch.bfloat16, device='cuda')
                L['ring_v'] = torch.zeros(B, R, D, dtype=torch.bfloat16, device='cuda')
                L['ring_g'] = torch.zeros(B, R, device='cuda')
                L['ring_u'] = torch.zeros(B, R, DI, dtype=torch.bfloat16, device='cuda') if kind == 'csa' else None
                for p in range(nb0 * m, T0):
                    L['ring_k'][:, p % R] = L['rk'][:, p]
                    L['ring_v'][:, p % R] = L['rv'][:, p]
                    L['ring_g'][:, p % R] = L['g'][:, p]
                    if kind == 'csa':
                        L['ring_u'][:, p % R] = L['ru'][:, p]
                calls.append(v4.csa_compress(L['ring_g'], L['bias'], 0, L['ring_k'], L['ring_v'], L['ek'], L['ev'],
                                             L['ring_u'], L['ik'], prepare=True, block_end=pos_b))
                if kind == 'csa':
                    ip, isc = F.mxfp4_quantize(q['iq'])
                    L['iq_all'], L['iqs_all'], L['w_all'] = dev(ip), dev(isc), dev(q['w'])
                    L['iq'] = torch.empty(B, 1, HI, DI // 2, dtype=torch.uint8, device='cuda')
                    L['iqs'] = torch.empty(B, 1, HI, DI // 32, dtype=torch.uint8, device='cuda')
                    L['w'] = torch.empty(B, 1, HI, device='cuda')
                    L['idx'] = torch.zeros(B, 1, K, dtype=torch.int32, device='cuda')
                    calls.append(v4.lightning_index_topk(pos, L['iq'], L['w'], L['ik'], K, m, iq_scale=L['iqs'],
                                                         out_idx=L['idx'], workspace=wsi, prepare=True))
                    calls.append(v4.sparse_window_attn(L['q'], pos, L['ek'], L['ev'], m, L['wk'], L['wv'], W,
                                                       L['idx'], o=L['o'], workspace=wsa, prepare=True,
                                                       append_k=L['ak'], append_v=L['av']))
                else:
                    calls.append(v4.hca_attn(L['q'], pos, L['ek'], L['ev'], m, L['wk'], L['wv'], W, o=L['o'],
                                             workspace=wsa, prepare=True, append_k=L['ak'], append_v=L['av']))
            L['calls'] = calls
            layers.append(L)
    torch.cuda.synchronize()

    def step_inputs(i):
        """The program's own work before step i (eager): the token's raw rows into the raw
        rings and the append buffers, the queries, the position."""
        t = T0 + i
        pos.fill_(t)
        for L in layers:
            L['q'].copy_(L['q_all'][:, i:i + 1])
            L['ak'].copy_(L['rk'][:, t:t + 1])
            L['av'].copy_(L['rv'][:, t:t + 1])
            if 'R' in L:
                L['ring_k'][:, t % L['R']] = L['rk'][:, t]
                L['ring_v'][:, t % L['R']] = L['rv'][:, t]
                L['ring_g'][:, t % L['R']] = L['g'][:, t]
                if L['kind'] == 'csa':
                    L['ring_u'][:, t % L['R']] = L['ru'][:, t]
            if L['kind'] == 'csa':
                L['iq'].copy_(L['iq_all'][:, i:i + 1])
                L['iqs'].copy_(L['iqs_all'][:, i:i + 1])
                L['w'].copy_(L['w_all'][:, i:i + 1])

    def step():
        for L in layers:
            for c in L['calls']:
                c()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        step_inputs(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        step()
    print('oracle caches', flush=True)
    ora = [_oracle_layer(kind, raws[l]) for l, kind in enumerate(KINDS)]
    for i in range(S):
        t = T0 + i
        with torch.cuda.stream(s):
            step_inputs(i)
            if i < 2:
                step()       # eager (rewrites the same rows as the replay below)
        torch.cuda.synchronize()
        eager = [L['o'].clone() for L in layers] if i < 2 else None
        for L in layers:
            L['o'].fill_(float('nan'))
        torch.cuda.synchronize()
        print(f'stack step {i} (t = {t}): replay', flush=True)
        graph.replay()
        torch.cuda.synchronize()
        if eager is not None:
            assert all(torch.equal(L['o'], e) for L, e in zip(layers, eager)), f'step {i}: replay differs from eager'
        for l, (L, kind) in enumerate(zip(layers, KINDS)):
            o = L['o'].cpu().numpy()
            O, q = ora[l], qs[l]
            for b in range(B):
                qr = q['q'][b, i]
                what = f'step {i} t={t} layer {l} ({kind}) b{b}'
                if kind == 'win':
                    ro, _ = OM.window_query(qr, t, O['dwk'][b], O['dwv'][b], W)
                elif kind == 'hca':
                    ro, _ = OM.hca_query(qr, t, O['dk'][b], O['dv'][b], O['dwk'][b], O['dwv'][b], M_OF[kind], W)
                else:
                    diq = F.mxfp4_dequantize(*F.mxfp4_quantize(q['iq'][b, i]))
                    ro, _, sel, scores = OM.csa_query(qr, t, diq, q['w'][b, i], O['dik'][b], O['dk'][b], O['dv'][b],
                                                      O['dwk'][b], O['dwv'][b], M_OF[kind], K, W)
                    g_sel = L['idx'][b, 0].cpu().numpy()
                    n_vis = OI.n_visible(t, M_OF[kind], O['dik'].shape[1])
                    assert_topk(g_sel, scores, n_vis, K, what)
                    if not np.array_equal(np.sort(g_sel), np.sort(sel)):
                        ro, _ = OA.attend_query(qr, t, g_sel, O['dk'][b], O['dv'][b], O['dwk'][b], O['dwv'][b], W)
                assert_close_rms(o[b, 0], ro, TOL_BF16, what)
    # what the graph wrote: the entries of the blocks completed during the steps, and the window rows
    for l, (L, kind) in enumerate(zip(layers, KINDS)):
        O = ora[l]
        for b in range(B):
            if kind != 'win':
                m = M_OF[kind]
                new = np.arange(T0 // m, TT // m)
                assert len(new) > 0
                assert_kv_rows(*kv_planes(L['ek'], b, new), O['k32'][b, new], f'layer {l} new K entries b{b}')
                assert_kv_rows(*kv_planes(L['ev'], b, new), O['v32'][b, new], f'layer {l} new V entries b{b}')
            wpos = np.arange(TT - W, TT)
            assert_kv_rows(*kv_planes(L['wk'], b, wpos % W), O['wk32'][b, wpos], f'layer {l} window K b{b}')
            assert_kv_rows(*kv_planes(L['wv'], b, wpos % W), O['wv32'][b, wpos], f'layer {l} window V b{b}')
