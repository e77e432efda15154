"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the benchmark.

This module holds none of the method's arithmetic: it draws random floats with
the shapes and distributions of the five workloads (raw tokens, gate logits,
positional biases, entry-level keys and values, queries, indexer queries and
weights) and rounds them to the input precision (bfloat16 via torch where a
workload says the activations are bf16). Quantisation into cache formats,
compression, scoring and attention are done elsewhere, on each side separately.

Every tensor comes from its own child of a numpy SeedSequence, keyed by the
case seed and the tensor's name, so any tensor can be regenerated alone.
"""

import hashlib

import numpy as np
import torch

ROPE_BASE = 10000.0


def _rng(seed, name):
    h = int.from_bytes(hashlib.sha256(name.encode()).digest()[:4], 'little')
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), h])))


def normal(seed, name, shape, std=1.0, outlier_frac=0.0, outlier_mult=20.0):
    """N(0, std^2) float32; a Bernoulli(outlier_frac) mask of elements is multiplied by outlier_mult."""
    g = _rng(seed, name)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0:
        mask = g.random(size=shape, dtype=np.float32) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return x


def uniform(seed, name, shape, lo=0.0, hi=1.0):
    g = _rng(seed, name)
    return (lo + (hi - lo) * g.random(size=shape, dtype=np.float32)).astype(np.float32)


def to_bf16_values(x):
    """Round float32 values to bfloat16 (torch's round-to-nearest-even); returned as float32."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def raw_tokens(seed, B, T, D, m, d_I=0, std=1.0, bf16=True, t0=0, prefix='layer'):
    """Raw per-token inputs of one layer for positions [t0, t0+T).

    raw_k/raw_v [B, T, D], gate [B, T] ~ N(0,1), pos_bias [m] ~ N(0, 0.1^2),
    raw_ik [B, T, d_I] (when d_I > 0). The position range is part of each
    tensor's name.
    """
    name = f'{prefix}/{t0}:{T}'
    out = {
        'raw_k': normal(seed, name + '/raw_k', (B, T, D), std),
        'raw_v': normal(seed, name + '/raw_v', (B, T, D), std),
        'gate': normal(seed, name + '/gate', (B, T)),
        'pos_bias': normal(seed, f'{prefix}/pos_bias/{m}', (m,), 0.1),
    }
    if d_I:
        out['raw_ik'] = normal(seed, name + '/raw_ik', (B, T, d_I), std)
    if bf16:
        for kk in ('raw_k', 'raw_v', 'raw_ik'):
            if kk in out:
                out[kk] = to_bf16_values(out[kk])
    return out


def queries(seed, B, Tq, H_q, D, H_I=0, d_I=0, std=1.0, idx_std=None, outlier_frac=0.0,
            bf16=True, prefix='q'):
    """Attention queries q [B, Tq, H_q, D], indexer queries iq [B, Tq, H_I, d_I], weights w ~ U(0,1)."""
    out = {'q': normal(seed, prefix + '/q', (B, Tq, H_q, D), std, outlier_frac)}
    if bf16:
        out['q'] = to_bf16_values(out['q'])
    if H_I:
        out['iq'] = normal(seed, prefix + '/iq', (B, Tq, H_I, d_I),
                           std if idx_std is None else idx_std, outlier_frac)
        out['w'] = uniform(seed, prefix + '/w', (B, Tq, H_I))
    return out


def entries(seed, B, N, D, d_I=0, W=128, outlier_frac=0.0, prefix='ent'):
    """Entry-level keys/values [B, N, D], window rows [B, W, D] and indexer keys [B, N, d_I]."""
    out = {
        'ent_k': normal(seed, prefix + '/k', (B, N, D), 1.0, outlier_frac),
        'ent_v': normal(seed, prefix + '/v', (B, N, D), 1.0, outlier_frac),
        'win_k': normal(seed, prefix + '/wk', (B, W, D), 1.0, outlier_frac),
        'win_v': normal(seed, prefix + '/wv', (B, W, D), 1.0, outlier_frac),
    }
    if d_I:
        out['ik'] = normal(seed, prefix + '/ik', (B, N, d_I), 1.0, outlier_frac)
    return out


def plant(seed, ik, iq, w, n_plant=64, c=8.0, noise=0.1, prefix='plant'):
    """Overwrite n_plant random indexer keys per batch element with keys aligned to the query.

    Planted key = c * sqrt(d_I) * unit(sum_h w_h iq_h) + noise * N(0,1). Returns the
    planted ids [B, n_plant] (sorted). Uses only the first query of each batch element.
    """
    B, N, d_I = ik.shape
    g = _rng(seed, prefix + '/ids')
    ids = np.stack([np.sort(g.choice(N, size=n_plant, replace=False)) for _ in range(B)])
    for b in range(B):
        direction = (w[b, 0][:, None].astype(np.float64) * iq[b, 0].astype(np.float64)).sum(0)
        direction /= np.linalg.norm(direction)
        nz = normal(seed, f'{prefix}/noise/{b}', (n_plant, d_I), noise)
        ik[b, ids[b]] = (c * np.sqrt(d_I) * direction[None, :] + nz).astype(np.float32)
    return ids


# ------------------------------------------------------------ workloads ----
# Shapes of the five workloads (B: batch, T: context, m: compression ratio,
# k: selected entries, W: window, H_q query heads sharing one KV head of dim D,
# H_I x d_I indexer heads).

WORKLOADS = {
    'c0_csa_fp32_4k': dict(B=1, T=4096, Tq=16, D=128, H_q=16, m=4, H_I=4, d_I=64, k=64, W=128,
                           kv='f32', ik='f32', act='f32'),
    'c1_csa_64k': dict(B=8, T=65536, Tq=1, D=192, H_q=64, m=4, H_I=64, d_I=128, k=512, W=128,
                       kv='e4m3_bf16', ik='mxfp4', act='bf16'),
    'c2_hca_1m': dict(B=4, T=1048576, Tq=1, D=192, H_q=64, m=128, k=None, W=128,
                      kv='e4m3_bf16', act='bf16'),
    'c3_csa_1m': dict(B=4, T=1048576, Tq=1, D=192, H_q=64, m=4, H_I=64, d_I=128, k=1024, W=128,
                      kv='e4m3_bf16', ik='mxfp4', act='bf16'),
    'c4_prefill_128k': dict(B=1, T0=131072, T1=8192, D=192, H_q=64, m_csa=4, m_hca=128, H_I=64,
                            d_I=128, k=1024, W=128, layers=('csa', 'hca', 'csa', 'hca'),
                            kv='e4m3_bf16', ik='mxfp4', act='bf16'),
}


def c0(seed=0):
    """fp32 CSA layer, 4,096 tokens, decode of the last 16 positions."""
    cfg = WORKLOADS['c0_csa_fp32_4k']
    s = 1.0 / np.sqrt(128.0)
    out = raw_tokens(seed, 1, cfg['T'], cfg['D'], cfg['m'], cfg['d_I'], std=s, bf16=False)
    out['raw_ik'] = normal(seed, 'layer/raw_ik_c0', (1, cfg['T'], cfg['d_I']), 1.0 / np.sqrt(64.0))
    out.update(queries(seed, 1, cfg['Tq'], cfg['H_q'], cfg['D'], cfg['H_I'], cfg['d_I'], std=s,
                       idx_std=1.0 / np.sqrt(64.0), bf16=False))
    out['q_pos'] = np.arange(cfg['T'] - cfg['Tq'], cfg['T'], dtype=np.int64)[None, :]
    return cfg, out


def entry_decode(seed, B, N, t, D, H_q, H_I, d_I, W=128, outlier_frac=0.01, n_plant=0):
    """Entry-level decode case (the shape of the 64K and 1M CSA workloads)."""
    out = entries(seed, B, N, D, d_I, W, outlier_frac if n_plant == 0 else 0.0)
    out.update(queries(seed, B, 1, H_q, D, H_I, d_I, outlier_frac=outlier_frac))
    out['q_pos'] = np.full((B, 1), t, np.int64)
    if n_plant:
        out['planted'] = plant(seed, out['ik'], out['iq'], out['w'], n_plant)
    return out


def c1(seed=1):
    cfg = WORKLOADS['c1_csa_64k']
    N = cfg['T'] // cfg['m']
    return cfg, entry_decode(seed, cfg['B'], N, cfg['T'] - 1, cfg['D'], cfg['H_q'], cfg['H_I'],
                             cfg['d_I'], cfg['W'], 0.01)


def c3(seed=3, B=None):
    cfg = WORKLOADS['c3_csa_1m']
    N = cfg['T'] // cfg['m']
    return cfg, entry_decode(seed, B or cfg['B'], N, cfg['T'] - 1, cfg['D'], cfg['H_q'], cfg['H_I'],
                             cfg['d_I'], cfg['W'], 0.01, n_plant=64)


def c2_batch(seed, b):
    """Raw tokens of batch element b of the 1M-token HCA workload (bf16 values)."""
    cfg = WORKLOADS['c2_hca_1m']
    return raw_tokens(seed * 1000 + b, 1, cfg['T'], cfg['D'], cfg['m'], 0, bf16=True)


def c2_queries(seed=2):
    cfg = WORKLOADS['c2_hca_1m']
    out = queries(seed, cfg['B'], 1, cfg['H_q'], cfg['D'])
    out['q_pos'] = np.full((cfg['B'], 1), cfg['T'] - 1, np.int64)
    return cfg, out


def c4_layer(seed, layer, T=None, t0=0):
    """Raw tokens of one layer of the chunked-prefill workload for positions [t0, t0+T)."""
    cfg = WORKLOADS['c4_prefill_128k']
    kind = cfg['layers'][layer]
    m = cfg['m_csa'] if kind == 'csa' else cfg['m_hca']
    T = cfg['T0'] + cfg['T1'] if T is None else T
    d_I = cfg['d_I'] if kind == 'csa' else 0
    return kind, raw_tokens(seed, 1, T, cfg['D'], m, d_I, bf16=True, t0=t0, prefix=f'c4/{layer}')


def c4_queries(seed, layer, T0=None, T1=None):
    """Queries of one prefill layer for the new tokens at positions T0 .. T0+T1-1."""
    cfg = WORKLOADS['c4_prefill_128k']
    T0 = cfg['T0'] if T0 is None else T0
    T1 = cfg['T1'] if T1 is None else T1
    out = queries(seed, 1, T1, cfg['H_q'], cfg['D'], cfg['H_I'], cfg['d_I'],
                  prefix=f'c4q/{layer}/{T0}:{T1}')
    out['q_pos'] = (T0 + np.arange(T1, dtype=np.int64))[None, :]
    return out


# ------------------------------------------------------- device-side draws ----
# The same recipes drawn with torch's generator on the GPU, for workloads too
# large to draw on the host quickly (the benchmark's caches). Still no method
# arithmetic: random floats, outlier masks and bf16 rounding of inputs only.

def _torch_gen(seed, name, device):
    h = int.from_bytes(hashlib.sha256(name.encode()).digest()[:4], 'little')
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 32) ^ h)
    return g


def gpu_normal(seed, name, shape, std=1.0, outlier_frac=0.0, outlier_mult=20.0, dtype=torch.float32,
               device='cuda'):
    g = _torch_gen(seed, name, device)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if outlier_frac > 0:
        mask = torch.rand(shape, generator=g, device=device) < outlier_frac
        x[mask] *= outlier_mult
    return x.to(dtype)


def gpu_uniform(seed, name, shape, device='cuda'):
    return torch.rand(shape, generator=_torch_gen(seed, name, device), device=device, dtype=torch.float32)


def gpu_plant(seed, ik, iq, w, n_plant=64, c=8.0, noise=0.1):
    """Device version of plant(): ik [B, N, d_I] float32 (modified), iq [B, 1, H, d_I], w [B, 1, H]."""
    B, N, d_I = ik.shape
    g = _torch_gen(seed, 'plant/ids', ik.device)
    ids = torch.stack([torch.randperm(N, generator=g, device=ik.device)[:n_plant].sort().values for _ in range(B)])
    for b in range(B):
        d = (w[b, 0][:, None].double() * iq[b, 0].double()).sum(0)
        d = d / d.norm()
        nz = gpu_normal(seed, f'plant/noise/{b}', (n_plant, d_I), noise, device=ik.device)
        ik[b, ids[b]] = (c * d_I ** 0.5 * d[None, :]).float() + nz
    return ids
