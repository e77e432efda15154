// lightning_index_topk: score every visible compressed entry per query and
// keep the k best.
//
// [webconsulting.at, "DeepSeek V4-Pro: Architektur, KV-Cache-Kompression und
// Hyper-Connections im Detail", section "Kompression und Selektion"]: the
// indexer scans the compressed entries at low precision and forwards the 1,024
// most relevant to the CSA layers. [chaosnode.de, "DeepSeek-V4: 1 Million
// Token Context endlich nutzbar", section "Hybrid Attention: CSA und HCA"]: top-k
// compressed blocks per query, indexer in FP4. The score formula is a reading
// (the pages give none): I_e = sum_h w_h * max(0, q_h . u_e).
//
// Structure (one launch):
//  1. Workgroup (chunk, query) scores `chunk` consecutive entries. MXFP4 keys:
//     V_MFMA_SCALE_F32_16X16X128_F8F6F4 with the indexer heads as M (16 per
//     tile), 16 keys as N and the whole 128-dim key as K; the E8M0 block
//     scales ride in the instruction. Each lane loads one 16-byte quarter of
//     one key row, so a wave reads 1 KB of contiguous key bytes per tile.
//     The ReLU-weighted head sum is taken in the accumulator lanes.
//  2. The chunk keeps its local top-s candidates: a two-pass LDS radix
//     histogram (top 16 bits of the order-preserving score key) finds a
//     threshold; every entry at or above it is written, in index order, to the
//     chunk's candidate region with the threshold as the region's lower bound.
//  3. The last workgroup of a query to arrive (device-scope counter) merges:
//     radix-selects the k-th key over the candidates, checks that no chunk
//     could have withheld an entry at or above it (lower bound > k-th key), and
//     writes the selection in ascending id order. If a chunk could have
//     withheld one (clustered winners, huge ties, region overflow) the merge
//     falls back to an exact radix select that rescores every visible entry.

#include "common.hpp"

namespace v4a {

constexpr int IT = 256;  // threads per workgroup (4 waves)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct IdxSmem {
    uint32_t hist[256];
    uint32_t scan[IT / 64 + 1];
    int misc[8];
};

__device__ __forceinline__ int64_t visible_entries(const IndexPlan &p, int q) {
    int64_t t = p.q_pos[q];
    if (t < 0) return 0;
    int64_t n = (t + 1) / p.m;
    return n < p.keys.rows ? n : p.keys.rows;
}

// Inclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ uint32_t block_scan(uint32_t v, IdxSmem &sm, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        uint32_t y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
    }
    __syncthreads();
    if (lane == 63) sm.scan[wave] = x;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < IT / 64; ++w) {
        uint32_t t = sm.scan[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    *total = all;
    return x + before;
}

// Largest bin b with sum(hist[b..255]) >= need. Returns b; *above = sum(hist[b+1..255]).
__device__ int find_bin(IdxSmem &sm, uint32_t need, uint32_t *above) {
    const int tid = threadIdx.x;
    uint32_t total;
    uint32_t suf = block_scan(sm.hist[255 - tid], sm, &total);  // thread t: bins 255-t .. 255
    uint32_t excl = suf - sm.hist[255 - tid];
    __syncthreads();
    if (suf >= need && excl < need) {
        sm.misc[0] = 255 - tid;
        sm.misc[1] = (int)excl;
    }
    __syncthreads();
    int b = sm.misc[0];
    *above = (uint32_t)sm.misc[1];
    __syncthreads();
    return b;
}

// ------------------------------------------------------------- scoring ----

template <int NT>
__device__ __forceinline__ float head_sum(const v8i (&A)[4], uint32_t sA, const v8i &B, uint32_t sB,
                                          const float (&wv)[4][4]) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    float s = 0.f;
    v4f acc;
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B, z, 4, 4, 0, sA, 0, sB);
#pragma unroll
    for (int j = 0; j < 4; ++j) s += wv[0][j] * __builtin_fmaxf(acc[j], 0.f);
    if (NT > 1) {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B, z, 4, 4, 1, sA, 0, sB);
#pragma unroll
        for (int j = 0; j < 4; ++j) s += wv[1][j] * __builtin_fmaxf(acc[j], 0.f);
    }
    if (NT > 2) {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B, z, 4, 4, 2, sA, 0, sB);
#pragma unroll
        for (int j = 0; j < 4; ++j) s += wv[2][j] * __builtin_fmaxf(acc[j], 0.f);
    }
    if (NT > 3) {
        acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[3], B, z, 4, 4, 3, sA, 0, sB);
#pragma unroll
        for (int j = 0; j < 4; ++j) s += wv[3][j] * __builtin_fmaxf(acc[j], 0.f);
    }
    return s;
}

constexpr int MX_BATCH = 8;  // key tiles whose loads are in flight together per wave

// Scores of entries [c0, c0+cnt) -> skey[0..cnt) (order-preserving keys).
template <int NT>
__device__ void score_chunk_mx(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const uint8_t *iq = (const uint8_t *)p.iq + (size_t)q * p.H * 64;
    const uint8_t *iqs = p.iq_scale + (size_t)q * p.H * 4;
    const float *w = p.w + (size_t)q * p.H;
    v8i A[4];
    uint32_t sA = 0;
    float wv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v4i v = {0, 0, 0, 0};
        uint32_t sc = 0;
        if (i < NT) {
            v = *(const v4i *)(iq + (16 * i + col) * 64 + 16 * grp);
            sc = iqs[(16 * i + col) * 4 + grp];
        }
        A[i] = (v8i){v[0], v[1], v[2], v[3], 0, 0, 0, 0};
        sA |= sc << (8 * i);
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[i][j] = (i < NT) ? w[16 * i + 4 * grp + j] : 0.f;
    }
    const char *kc = p.keys.e2m1 + (int64_t)b * p.keys.e2m1_bs + 16 * grp;
    const char *ks = p.keys.e8m0 + (int64_t)b * p.keys.e8m0_bs + grp;
    const int64_t krs = p.keys.e2m1_rs, srs = p.keys.e8m0_rs;
    const int ntiles = (cnt + 15) >> 4;
    for (int t0 = wave; t0 < ntiles; t0 += 4 * MX_BATCH) {
        v4i kv[MX_BATCH];
        uint32_t sB[MX_BATCH];
#pragma unroll
        for (int u = 0; u < MX_BATCH; ++u) {
            const int tile = t0 + 4 * u;
            int r = tile * 16 + col;
            r = r < cnt ? r : 0;  // tail lanes reload row c0 (always valid); masked below
            kv[u] = __builtin_nontemporal_load((const v4i *)(kc + (c0 + r) * krs));
            sB[u] = (uint8_t)__builtin_nontemporal_load((const char *)(ks + (c0 + r) * srs));
        }
#pragma unroll
        for (int u = 0; u < MX_BATCH; ++u) {
            const int tile = t0 + 4 * u;
            if (tile >= ntiles) break;
            v8i B = {kv[u][0], kv[u][1], kv[u][2], kv[u][3], 0, 0, 0, 0};
            float s = head_sum<NT>(A, sA, B, sB[u], wv);
            s += __shfl_xor(s, 16, 64);
            s += __shfl_xor(s, 32, 64);
            const int r = tile * 16 + col;
            if (grp == 0 && r < cnt) skey[r] = score_key(s);
        }
    }
}

constexpr int F32_MAX_H = 16;

// float32 keys: one entry per thread, dot products in float64.
__device__ void score_chunk_f32(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey,
                                const float *sq) {
    const int H = p.H, dI = p.dI;
    const float *w = p.w + (size_t)q * H;
    for (int r = threadIdx.x; r < cnt; r += IT) {
        const float *key = (const float *)(p.keys.f32 + (int64_t)b * p.keys.f32_bs + (c0 + r) * p.keys.f32_rs);
        double acc[F32_MAX_H];
#pragma unroll
        for (int h = 0; h < F32_MAX_H; ++h) acc[h] = 0.0;
        for (int j = 0; j < dI; j += 4) {
            float4 kv = *(const float4 *)(key + j);
#pragma unroll
            for (int h = 0; h < F32_MAX_H; ++h) {
                if (h < H) {
                    const float *qq = sq + h * dI + j;
                    acc[h] += (double)qq[0] * kv.x;
                    acc[h] += (double)qq[1] * kv.y;
                    acc[h] += (double)qq[2] * kv.z;
                    acc[h] += (double)qq[3] * kv.w;
                }
            }
        }
        double s = 0.0;
#pragma unroll
        for (int h = 0; h < F32_MAX_H; ++h)
            if (h < H) s += (double)w[h] * __builtin_fmax(acc[h], 0.0);
        skey[r] = score_key((float)s);
    }
}

template <int MODE>  // 0: f32 keys, 1..4: MXFP4 with MODE head tiles
__device__ __forceinline__ void score_chunk(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey,
                                            const float *sq) {
    if (MODE == 0) score_chunk_f32(p, q, b, c0, cnt, skey, sq);
    else score_chunk_mx<MODE>(p, q, b, c0, cnt, skey);
}

// ---------------------------------------------------- chunk candidates ----

// Keep the chunk's entries whose key's top 16 bits reach the s-th largest.
__device__ void chunk_emit(const IndexPlan &p, int q, int chunk, int64_t c0, int cnt, int s_want,
                           const uint32_t *skey, IdxSmem &sm) {
    const int tid = threadIdx.x;
    const size_t rid = (size_t)q * p.n_chunks + chunk;
    uint32_t thr = 0;  // emit keys >= thr
    if (cnt > s_want) {
        for (int i = tid; i < 256; i += IT) sm.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < cnt; i += IT) atomicAdd(&sm.hist[skey[i] >> 24], 1u);
        __syncthreads();
        uint32_t above1;
        const int b1 = find_bin(sm, (uint32_t)s_want, &above1);
        for (int i = tid; i < 256; i += IT) sm.hist[i] = 0;
        __syncthreads();
        for (int i = tid; i < cnt; i += IT)
            if ((int)(skey[i] >> 24) == b1) atomicAdd(&sm.hist[(skey[i] >> 16) & 255u], 1u);
        __syncthreads();
        uint32_t above2;
        const int b2 = find_bin(sm, (uint32_t)s_want - above1, &above2);
        thr = ((uint32_t)b1 << 24) | ((uint32_t)b2 << 16);
    }
    // compaction in index order: thread t owns entries [t*per, t*per + per)
    const int per = (p.chunk + IT - 1) / IT;
    const int lo = tid * per;
    uint32_t mine = 0;
    for (int i = lo; i < lo + per && i < cnt; ++i) mine += skey[i] >= thr;
    uint32_t total;
    uint32_t off = block_scan(mine, sm, &total) - mine;
    uint32_t *meta = p.meta + rid * 2;
    if (total > (uint32_t)p.region_cap) {
        if (tid == 0) {
            meta[0] = 0xFFFFFFFFu;  // overflow: the merge falls back
            meta[1] = 0xFFFFFFFFu;
        }
        return;
    }
    uint32_t *rk = p.reg_key + rid * p.region_cap;
    int32_t *ri = p.reg_idx + rid * p.region_cap;
    for (int i = lo; i < lo + per && i < cnt; ++i) {
        if (skey[i] >= thr) {
            rk[off] = skey[i];
            ri[off] = (int32_t)(c0 + i);
            ++off;
        }
    }
    if (tid == 0) {
        meta[0] = total;
        meta[1] = thr;
    }
}

// ------------------------------------------------------------- merge ----

constexpr int REG_CAND = 32;  // candidates a merge thread keeps in registers

template <int MODE>
__device__ void exact_fallback(const IndexPlan &p, int q, int b, int64_t nvis, int kk, uint32_t *skey,
                               const float *sq, IdxSmem &sm) {
    // Radix select over every visible entry, rescoring chunk by chunk.
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0, need = (uint32_t)kk;
    for (int d = 3; d >= 0; --d) {
        for (int i = tid; i < 256; i += IT) sm.hist[i] = 0;
        __syncthreads();
        for (int64_t c0 = 0; c0 < nvis; c0 += p.chunk) {
            const int cnt = (int)((nvis - c0) < p.chunk ? (nvis - c0) : p.chunk);
            score_chunk<MODE>(p, q, b, c0, cnt, skey, sq);
            __syncthreads();
            for (int i = tid; i < cnt; i += IT)
                if ((skey[i] & mask) == prefix) atomicAdd(&sm.hist[(skey[i] >> (8 * d)) & 255u], 1u);
            __syncthreads();
        }
        uint32_t above;
        const int bin = find_bin(sm, need, &above);
        need -= above;
        prefix |= (uint32_t)bin << (8 * d);
        mask |= 255u << (8 * d);
    }
    // kth key = prefix; take every key > prefix and the first `need` equal ones.
    int32_t *oidx = p.out_idx + (size_t)q * p.k;
    float *osc = p.out_score ? p.out_score + (size_t)q * p.k : nullptr;
    uint32_t written = 0, ties = 0;
    const int per = (p.chunk + IT - 1) / IT;
    for (int64_t c0 = 0; c0 < nvis; c0 += p.chunk) {
        const int cnt = (int)((nvis - c0) < p.chunk ? (nvis - c0) : p.chunk);
        score_chunk<MODE>(p, q, b, c0, cnt, skey, sq);
        __syncthreads();
        const int lo = threadIdx.x * per;
        uint32_t nt = 0;
        for (int i = lo; i < lo + per && i < cnt; ++i) nt += skey[i] == prefix;
        uint32_t tot_t;
        uint32_t tie_before = ties + block_scan(nt, sm, &tot_t) - nt;
        uint32_t ns = 0;
        {
            uint32_t tb = tie_before;
            for (int i = lo; i < lo + per && i < cnt; ++i) {
                if (skey[i] > prefix) ++ns;
                else if (skey[i] == prefix) ns += (tb++ < need);
            }
        }
        uint32_t tot_s;
        uint32_t pos = written + block_scan(ns, sm, &tot_s) - ns;
        {
            uint32_t tb = tie_before;
            for (int i = lo; i < lo + per && i < cnt; ++i) {
                bool take = skey[i] > prefix;
                if (skey[i] == prefix) take = (tb++ < need);
                if (take) {
                    oidx[pos] = (int32_t)(c0 + i);
                    if (osc) osc[pos] = key_score(skey[i]);
                    ++pos;
                }
            }
        }
        written += tot_s;
        ties += tot_t;
        __syncthreads();
    }
    for (int i = kk + tid; i < p.k; i += IT) {
        oidx[i] = -1;
        if (osc) osc[i] = 0.f;
    }
}

template <int MODE>
__device__ void merge(const IndexPlan &p, int q, int b, int64_t nvis, uint32_t *skey, const float *sq,
                      IdxSmem &sm) {
    const int tid = threadIdx.x;
    const int kk = (int)(nvis < p.k ? nvis : p.k);
    int32_t *oidx = p.out_idx + (size_t)q * p.k;
    float *osc = p.out_score ? p.out_score + (size_t)q * p.k : nullptr;
    if (kk == 0) {
        for (int i = tid; i < p.k; i += IT) {
            oidx[i] = -1;
            if (osc) osc[i] = 0.f;
        }
        return;
    }
    // thread t owns chunks [t*cpt, t*cpt + cpt) (in order)
    const int cpt = (p.n_chunks + IT - 1) / IT;
    const int cA = tid * cpt, cB = min(cA + cpt, p.n_chunks);
    const uint32_t *meta = p.meta + (size_t)q * p.n_chunks * 2;
    const uint32_t *rk = p.reg_key + (size_t)q * p.n_chunks * p.region_cap;
    const int32_t *ri = p.reg_idx + (size_t)q * p.n_chunks * p.region_cap;
    int bad = 0;
    uint32_t mycnt = 0;
    for (int c = cA; c < cB; ++c) {
        uint32_t n = meta[2 * c];
        if (n == 0xFFFFFFFFu) bad = 1;
        else mycnt += n;
    }
    const bool in_regs = (cB - cA == 1) && mycnt <= REG_CAND;
    uint32_t keys[REG_CAND];
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) keys[i] = (i < (int)mycnt) ? rk[(size_t)cA * p.region_cap + i] : 0u;
    }
    if (__syncthreads_or(bad)) {
        exact_fallback<MODE>(p, q, b, nvis, kk, skey, sq, sm);
        return;
    }
    // radix select of the kk-th largest candidate key
    uint32_t prefix = 0, mask = 0, need = (uint32_t)kk;
    for (int d = 3; d >= 0; --d) {
        for (int i = tid; i < 256; i += IT) sm.hist[i] = 0;
        __syncthreads();
        const int sh = 8 * d;
        if (in_regs) {
#pragma unroll
            for (int i = 0; i < REG_CAND; ++i)
                if (i < (int)mycnt && (keys[i] & mask) == prefix) atomicAdd(&sm.hist[(keys[i] >> sh) & 255u], 1u);
        } else {
            for (int c = cA; c < cB; ++c) {
                const uint32_t n = meta[2 * c];
                for (uint32_t i = 0; i < n; ++i) {
                    const uint32_t kx = rk[(size_t)c * p.region_cap + i];
                    if ((kx & mask) == prefix) atomicAdd(&sm.hist[(kx >> sh) & 255u], 1u);
                }
            }
        }
        __syncthreads();
        uint32_t above;
        const int bin = find_bin(sm, need, &above);
        need -= above;
        prefix |= (uint32_t)bin << sh;
        mask |= 255u << sh;
    }
    const uint32_t kth = prefix;
    // a chunk whose emitted lower bound lies above the k-th key may have withheld winners
    int sat = 0;
    for (int c = cA; c < cB; ++c) sat |= meta[2 * c + 1] > kth;
    if (__syncthreads_or(sat)) {
        exact_fallback<MODE>(p, q, b, nvis, kk, skey, sq, sm);
        return;
    }
    // emit: keys > kth, and the first `need` keys == kth in id order
    uint32_t nt = 0;
    if (in_regs) {
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) nt += (i < (int)mycnt) && keys[i] == kth;
    } else {
        for (int c = cA; c < cB; ++c)
            for (uint32_t i = 0; i < meta[2 * c]; ++i) nt += rk[(size_t)c * p.region_cap + i] == kth;
    }
    uint32_t tot;
    uint32_t tb = block_scan(nt, sm, &tot) - nt;
    uint32_t ns = 0;
    {
        uint32_t t2 = tb;
        for (int c = cA; c < cB; ++c)
            for (uint32_t i = 0; i < meta[2 * c]; ++i) {
                const uint32_t kx = rk[(size_t)c * p.region_cap + i];
                if (kx > kth) ++ns;
                else if (kx == kth) ns += (t2++ < need);
            }
    }
    uint32_t pos = block_scan(ns, sm, &tot) - ns;
    for (int c = cA; c < cB; ++c)
        for (uint32_t i = 0; i < meta[2 * c]; ++i) {
            const uint32_t kx = rk[(size_t)c * p.region_cap + i];
            bool take = kx > kth;
            if (kx == kth) take = (tb++ < need);
            if (take) {
                oidx[pos] = ri[(size_t)c * p.region_cap + i];
                if (osc) osc[pos] = key_score(kx);
                ++pos;
            }
        }
    for (int i = kk + tid; i < p.k; i += IT) {
        oidx[i] = -1;
        if (osc) osc[i] = 0.f;
    }
}

// ------------------------------------------------------------- kernel ----

template <int MODE>
__global__ __launch_bounds__(IT) void index_topk_kernel(IndexPlan p) {
    extern __shared__ uint32_t dyn[];
    __shared__ IdxSmem sm;
    __shared__ int last;
    uint32_t *skey = dyn;                                 // [chunk]
    float *sq = (float *)(dyn + p.chunk);                 // f32 mode: query [H][dI]
    const int chunk = blockIdx.x, q = blockIdx.y;
    const int b = q / p.Tq;
    const int tid = threadIdx.x;
    if (MODE == 0) {
        const float *iq = (const float *)p.iq + (size_t)q * p.H * p.dI;
        for (int i = tid; i < p.H * p.dI; i += IT) sq[i] = iq[i];
        __syncthreads();
    }
    const int64_t nvis = visible_entries(p, q);
    const int kk = (int)(nvis < p.k ? nvis : p.k);
    const int64_t c0 = (int64_t)chunk * p.chunk;
    const int cnt = (int)(nvis - c0 <= 0 ? 0 : (nvis - c0 < p.chunk ? nvis - c0 : p.chunk));
    if (cnt > 0) {
        score_chunk<MODE>(p, q, b, c0, cnt, skey, sq);
        __syncthreads();
        // every full chunk keeps enough that the union holds at least kk entries
        const int64_t n_active = (nvis + p.chunk - 1) / p.chunk;
        int s_want = p.s_local;
        const int64_t spread = (kk + (n_active > 1 ? n_active - 1 : 1) - 1) / (n_active > 1 ? n_active - 1 : 1);
        if (spread > s_want) s_want = (int)spread;
        if (s_want > cnt) s_want = cnt;
        chunk_emit(p, q, chunk, c0, cnt, s_want, skey, sm);
    } else if (tid == 0) {
        uint32_t *meta = p.meta + ((size_t)q * p.n_chunks + chunk) * 2;
        meta[0] = 0;
        meta[1] = 0;
    }
    // arrive; the last workgroup of this query merges
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(&p.counters[q], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last = (prev == (uint32_t)p.n_chunks - 1);
    }
    __syncthreads();
    if (!last) return;
    __threadfence();
    merge<MODE>(p, q, b, nvis, skey, sq, sm);
    __syncthreads();
    if (tid == 0) __hip_atomic_store(&p.counters[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

hipError_t launch_index(const IndexPlan &p, hipStream_t s) {
    dim3 grid(p.n_chunks, p.Q);
    size_t lds = (size_t)p.chunk * 4 + (p.keys.fmt == 0 ? (size_t)p.H * p.dI * 4 : 0);
    if (p.keys.fmt == 0) {
        hipLaunchKernelGGL(index_topk_kernel<0>, grid, dim3(IT), lds, s, p);
    } else {
        switch (p.H / 16) {
            case 1: hipLaunchKernelGGL(index_topk_kernel<1>, grid, dim3(IT), lds, s, p); break;
            case 2: hipLaunchKernelGGL(index_topk_kernel<2>, grid, dim3(IT), lds, s, p); break;
            case 3: hipLaunchKernelGGL(index_topk_kernel<3>, grid, dim3(IT), lds, s, p); break;
            default: hipLaunchKernelGGL(index_topk_kernel<4>, grid, dim3(IT), lds, s, p); break;
        }
    }
    return hipGetLastError();
}

}  // namespace v4a
