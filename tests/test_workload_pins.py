"""CPU checks of the synthetic workloads themselves (no GPU).

The 1M-token CSA decode workload plants 64 keys per sequence aligned with the
query's weighted indexer direction, so that its top-k parity check has known
winners. Here the oracle confirms, on the exact bytes the GPU receives (MXFP4
keys and query), that every planted key outscores every other key.
"""

import numpy as np

import synth
from oracle import formats as F
from oracle import indexer as I


def test_c3_planted_keys_win_after_mxfp4():
    cfg = synth.WORKLOADS['c3_csa_1m']
    B, N, H, dI = cfg['B'], cfg['T'] // cfg['m'], cfg['H_I'], cfg['d_I']
    # the same draws, in the same streams, as synth.c3 (entry_decode with planting)
    ik = synth.normal(3, 'ent/ik', (B, N, dI))
    q = synth.queries(3, B, 1, cfg['H_q'], cfg['D'], H, dI, outlier_frac=0.01)
    planted = synth.plant(3, ik, q['iq'], q['w'], 64)
    diq = F.mxfp4_dequantize(*F.mxfp4_quantize(q['iq']))
    for b in range(B):
        dk = F.mxfp4_dequantize(*F.mxfp4_quantize(ik[b]))
        s = I.index_scores(diq[b, 0], q['w'][b, 0], dk).astype(np.float32)
        mask = np.zeros(N, bool)
        mask[planted[b]] = True
        lo, hi = s[mask].min(), s[~mask].max()
        assert lo > hi, f'b{b}: a bulk key ({hi}) scores at or above a planted one ({lo})'
        top = I.topk_select(s, N, cfg['k'])
        assert set(planted[b].tolist()) <= set(top.tolist())
        del dk
