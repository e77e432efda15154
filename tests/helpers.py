"""Shared pieces of the GPU parity tests: moving oracle-encoded stores to the
device, and the comparison rules.

Comparison rules:
* float outputs: max |gpu - oracle| <= tol * RMS(oracle), tol = 2e-2 for the
  FP8/BF16 path and 1e-5 for the float32 path;
* top-k sets: with tau the oracle's k-th score and Band = {e : |I_e - tau| <=
  1e-6 |tau|}, the GPU set and the oracle set have min(k, n_vis) members and
  agree outside Band (members inside Band must still be visible ids);
* cache codes: equal, except where the oracle's float32 value sits within a
  relative 1e-6 of the rounding boundary between the two codes (then they may
  differ by one step). This applies to E4M3 codes (value x / scale), E2M1 codes
  (value x / 2^E) and BF16 RoPE dims (value x); FP8 row scales and E8M0 block
  exponents must be equal.
"""

import numpy as np
import torch

import long_context_attention_compress_amd as v4
from oracle import formats as F

TOL_BF16 = 2e-2
TOL_F32 = 1e-5
BAND = 1e-6


def dev(x, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def bf16_dev(x):
    """float32 values that are exactly bf16 -> a device bfloat16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).cuda()


def kv_store(enc, ring=0):
    """Oracle-encoded KV planes (numpy, [B, rows, ...]) -> KVStore on the GPU."""
    if 'f32' in enc:
        return v4.KVStore(v4.KV_F32, enc['f32'].shape[-1], ring, f32=dev(enc['f32']))
    nope = dev(enc['nope'])
    rope = dev(enc['rope'].view(np.int16))
    scale = dev(enc['scale'])
    return v4.KVStore(v4.KV_E4M3_BF16, nope.shape[-1] + 64, ring, nope=nope, rope=rope, scale=scale)


def ik_store(enc):
    if 'f32' in enc:
        return v4.IKStore(v4.IK_F32, enc['f32'].shape[-1], f32=dev(enc['f32']))
    return v4.IKStore(v4.IK_MXFP4, enc['e2m1'].shape[-1] * 2, e2m1=dev(enc['e2m1']), e8m0=dev(enc['e8m0']))


def host_kv(store):
    if store.fmt == v4.KV_F32:
        return {'f32': store.f32.cpu().numpy()}
    return {'nope': store.nope.cpu().numpy(), 'rope': store.rope.cpu().numpy().view(np.uint16),
            'scale': store.scale.cpu().numpy()}


def host_ik(store):
    if store.fmt == v4.IK_F32:
        return {'f32': store.f32.cpu().numpy()}
    return {'e2m1': store.e2m1.cpu().numpy(), 'e8m0': store.e8m0.cpu().numpy()}


def ring_rows(rows_by_pos, first_pos, ring):
    """Place rows for positions first_pos.. into a ring of `ring` slots (slot = pos % ring)."""
    B, n = rows_by_pos.shape[:2]
    out = np.zeros((B, ring) + rows_by_pos.shape[2:], rows_by_pos.dtype)
    for i in range(n):
        out[:, (first_pos + i) % ring] = rows_by_pos[:, i]
    return out


def assert_close_rms(got, ref, tol, what=''):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    rms = np.sqrt(np.mean(ref ** 2))
    err = np.abs(got - ref).max()
    assert np.all(np.isfinite(got)), f'{what}: non-finite output'
    assert err <= tol * rms, f'{what}: max err {err:.3e} > {tol} x RMS {rms:.3e} (ratio {err / rms:.3e})'
    print(f'[close] {what}: max err / RMS = {err / rms:.3e} (tolerance {tol})', flush=True)
    return err / rms


def assert_topk(gpu_idx, scores, n_vis, k, what=''):
    """gpu_idx [k] int; scores: the oracle's scores of the n_vis visible entries."""
    from oracle import indexer as I
    ref = I.topk_select(scores, n_vis, k)
    kk = min(k, n_vis)
    g = np.asarray(gpu_idx)
    assert np.all(g[kk:] == -1), f'{what}: padding'
    gs = g[:kk]
    assert np.all(np.diff(gs) > 0), f'{what}: ids not strictly ascending'
    assert np.all((gs >= 0) & (gs < n_vis)), f'{what}: id out of range'
    if kk == 0:
        return 0
    s32 = np.asarray(scores, np.float64)[:n_vis].astype(np.float32).astype(np.float64)
    tau = I.kth_score(scores, n_vis, k)
    band = np.abs(s32 - tau) <= BAND * abs(tau)
    G, O = set(gs.tolist()), set(ref[:kk].tolist())
    outside = lambda S: {e for e in S if not band[e]}
    assert outside(G) == outside(O), (f'{what}: sets differ outside the tie band: '
                                      f'gpu-only {sorted(outside(G) - outside(O))[:10]} '
                                      f'oracle-only {sorted(outside(O) - outside(G))[:10]}')
    return len(G ^ O)


def assert_codes_e4m3(got, ref_codes, ref_vals, what=''):
    """E4M3 codes equal except near a rounding boundary of the oracle's value."""
    got = np.asarray(got, np.uint8)
    ref = np.asarray(ref_codes, np.uint8)
    bad = got != ref
    if not bad.any():
        return 0
    v = np.asarray(ref_vals, np.float64)[bad]
    a, b = F.e4m3_decode(got[bad]), F.e4m3_decode(ref[bad])
    mid = (a + b) / 2
    near = np.abs(v - mid) <= 1e-6 * np.maximum(np.abs(v), 1e-30)
    assert near.all(), f'{what}: {int((~near).sum())} codes differ away from a rounding boundary'
    return int(bad.sum())


def _assert_boundary(got_vals, ref_vals, oracle_vals, what, kind):
    """Where the decoded values differ, the oracle's value must lie within 1e-6 (relative)
    of the midpoint between them (a rounding boundary)."""
    bad = got_vals != ref_vals
    bad &= ~(np.isnan(got_vals) & np.isnan(ref_vals))
    if not bad.any():
        return 0
    a, b, v = got_vals[bad], ref_vals[bad], np.asarray(oracle_vals, np.float64)[bad]
    mid = (a + b) / 2
    near = np.abs(v - mid) <= 1e-6 * np.maximum(np.abs(v), 1e-30)
    assert near.all(), (f'{what}: {int((~near).sum())} {kind} values differ away from a rounding boundary '
                        f'(first: got {a[~near][:3]}, oracle code {b[~near][:3]}, value {v[~near][:3]})')
    return int(bad.sum())


def assert_bf16_bits(got, ref_bits, ref_vals, what=''):
    """BF16 bit patterns equal except where the oracle's float32 value sits at a rounding boundary."""
    return _assert_boundary(F.bf16_decode(np.asarray(got).view(np.uint16)), F.bf16_decode(ref_bits),
                            ref_vals, what, 'BF16')


def assert_kv_rows(g_nope, g_rope, g_scale, x32, what=''):
    """Every plane of E4M3_BF16 rows written by the GPU against the oracle's encoding of its
    float32 rows x32 [..., D]: scales equal, E4M3 codes and BF16 RoPE dims by the boundary rule.
    Returns the number of boundary differences."""
    x32 = np.asarray(x32, np.float32)
    codes, rope_bits, scale = F.kv_quantize(x32)
    g_scale = np.asarray(g_scale, np.float32).reshape(scale.shape)
    same = (g_scale == scale) | (np.isnan(g_scale) & np.isnan(scale))
    assert same.all(), f'{what}: {int((~same).sum())} FP8 row scales differ'
    q = (x32[..., :codes.shape[-1]].reshape(scale.shape + (-1,)) / scale[..., None]).astype(np.float32)
    n = assert_codes_e4m3(np.asarray(g_nope), codes, q.reshape(codes.shape), f'{what} E4M3')
    n += assert_bf16_bits(np.asarray(g_rope), rope_bits, x32[..., codes.shape[-1]:], f'{what} RoPE')
    return n


def assert_ik_rows(g_e2m1, g_e8m0, u32, what=''):
    """MXFP4 indexer-key rows: E8M0 exponents equal, E2M1 codes by the boundary rule."""
    u32 = np.asarray(u32, np.float32)
    packed, scales = F.mxfp4_quantize(u32)
    assert np.array_equal(np.asarray(g_e8m0), scales), f'{what}: E8M0 exponents differ'
    d = u32.shape[-1]
    blk = u32.reshape(u32.shape[:-1] + (d // F.MX_BLOCK, F.MX_BLOCK)).astype(np.float64)
    vals = (blk / F.e8m0_decode(scales)[..., None]).reshape(u32.shape)
    return _assert_boundary(F.e2m1_decode(F.mxfp4_unpack(np.asarray(g_e2m1))), F.e2m1_decode(F.mxfp4_unpack(packed)),
                            vals, f'{what} E2M1', 'E2M1')


def kv_planes(store, b, rows):
    """Host copies of the planes of batch element b, rows `rows`, of a device KVStore."""
    r = torch.as_tensor(np.asarray(rows, np.int64), device=store.nope.device)
    return (store.nope[b].index_select(0, r).cpu().numpy(),
            store.rope[b].index_select(0, r).cpu().numpy().view(np.uint16),
            store.scale[b].index_select(0, r).cpu().numpy())
