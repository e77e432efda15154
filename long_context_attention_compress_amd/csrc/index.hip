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
// Structure (two launches on the caller's stream):
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
//  3. A merge kernel (one workgroup per query) radix-selects the k-th key over
//     the candidates held in registers, checks that no chunk could have
//     withheld an entry at or above it (lower bound > k-th key), and writes the
//     selection in ascending id order. If a chunk could have withheld one
//     (clustered winners, huge ties, region overflow) the merge falls back to
//     an exact radix select that rescores every visible entry.

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

// Inclusive prefix sum over a wave with DPP row shifts and row broadcasts
// (VALU only; no LDS round trips).
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
    // within each row of 16 lanes
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    // across rows: lane 15 of each row is broadcast into the following row(s)
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return x;
}

// Inclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ uint32_t block_scan(uint32_t v, IdxSmem &sm, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t x = wave_inclusive_scan(v);
    (void)lane;
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

// max(0, x) as one VALU op (IEEE maxNum: a quiet-NaN x gives 0). The compiler's
// fmaxf would first canonicalise x, doubling the epilogue's VALU work.
__device__ __forceinline__ float relu1(float x) {
    float r;
    asm("v_max_f32 %0, 0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Sum over the four 16-lane rows holding the same key column, on the VALU
// (gfx950 lane-swap instructions instead of LDS-routed shuffles).
__device__ __forceinline__ float sum_rows(float s) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

template <int NT>
__device__ __forceinline__ float head_sum(const v8i (&A)[4], uint32_t sA, const v4i &kv, uint32_t sB,
                                          const float (&wv)[4][4]) {
    const v4f z = {0.f, 0.f, 0.f, 0.f};
    const v8i B = {kv[0], kv[1], kv[2], kv[3], 0, 0, 0, 0};
    v4f acc[4];
    acc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[0], B, z, 4, 4, 0, sA, 0, sB);
    if (NT > 1) acc[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[1], B, z, 4, 4, 1, sA, 0, sB);
    if (NT > 2) acc[2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[2], B, z, 4, 4, 2, sA, 0, sB);
    if (NT > 3) acc[3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[3], B, z, 4, 4, 3, sA, 0, sB);
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) s = __builtin_fmaf(wv[i][j], relu1(acc[i][j]), s);
    return s;
}

constexpr int MX_BATCH = 4;  // key tiles per wave per batch; two batches are in flight

// Scores of entries [c0, c0+cnt) -> skey[0..cnt) (order-preserving keys).
// Wave w takes tiles w, w+4, w+8, ...; each lane loads one 16-byte quarter of
// one key row per tile, addressed as a uniform base plus a 32-bit offset, and
// the next batch's loads are issued before the current batch is consumed.
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
    const char *kbase = p.keys.e2m1 + (int64_t)b * p.keys.e2m1_bs + c0 * p.keys.e2m1_rs;
    const char *sbase = p.keys.e8m0 + (int64_t)b * p.keys.e8m0_bs + c0 * p.keys.e8m0_rs;
    const uint32_t krs = (uint32_t)p.keys.e2m1_rs, srs = (uint32_t)p.keys.e8m0_rs;
    const int ntiles = (cnt + 15) >> 4;
    constexpr int STRIDE = 4 * MX_BATCH;  // tiles per batch over the 4 waves
    v4i ka[MX_BATCH], kb[MX_BATCH];
    uint32_t sa[MX_BATCH], sb[MX_BATCH];
    auto issue = [&](v4i (&kv)[MX_BATCH], uint32_t (&sv)[MX_BATCH], int t0) {
#pragma unroll
        for (int u = 0; u < MX_BATCH; ++u) {
            int r = (t0 + 4 * u) * 16 + col;
            r = r < cnt ? r : cnt - 1;  // tail lanes reload the last valid row; masked below
            kv[u] = __builtin_nontemporal_load((const v4i *)(kbase + (uint32_t)r * krs + 16 * grp));
            sv[u] = (uint8_t)__builtin_nontemporal_load(sbase + (uint32_t)r * srs + grp);
        }
    };
    auto consume = [&](const v4i (&kv)[MX_BATCH], const uint32_t (&sv)[MX_BATCH], int t0) {
#pragma unroll
        for (int u = 0; u < MX_BATCH; ++u) {
            const int tile = t0 + 4 * u;
            if (tile >= ntiles) break;
            const float s = sum_rows(head_sum<NT>(A, sA, kv[u], sv[u], wv));
            const int r = tile * 16 + col;
            if (grp == 0 && r < cnt) skey[r] = score_key(s);
        }
    };
    int t = wave;
    issue(ka, sa, t);
    for (; t < ntiles; t += 2 * STRIDE) {
        if (t + STRIDE < ntiles) issue(kb, sb, t + STRIDE);
        consume(ka, sa, t);
        if (t + STRIDE >= ntiles) break;
        if (t + 2 * STRIDE < ntiles) issue(ka, sa, t + 2 * STRIDE);
        consume(kb, sb, t + STRIDE);
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

constexpr int REG_CAND = 32;  // candidates a merge thread holds in registers

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

// ------------------------------------------------------------ kernels ----

template <int MODE>
__global__ __launch_bounds__(IT) void index_score_kernel(IndexPlan p) {
    extern __shared__ uint32_t dyn[];
    __shared__ IdxSmem sm;
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
    if (cnt == 0) {
        if (tid == 0) {
            uint32_t *meta = p.meta + ((size_t)q * p.n_chunks + chunk) * 2;
            meta[0] = 0;
            meta[1] = 0;
        }
        return;
    }
    score_chunk<MODE>(p, q, b, c0, cnt, skey, sq);
    __syncthreads();
    // every full chunk keeps enough that the union holds at least kk entries
    const int64_t n_active = (nvis + p.chunk - 1) / p.chunk;
    int s_want = p.s_local;
    const int64_t div = n_active > 1 ? n_active - 1 : 1;
    const int64_t spread = (kk + div - 1) / div;
    if (spread > s_want) s_want = (int)spread;
    if (s_want > cnt) s_want = cnt;
    chunk_emit(p, q, chunk, c0, cnt, s_want, skey, sm);
}

// One workgroup per query. The chunks' candidates are taken in chunk order
// (ascending entry ids) and split into equal contiguous runs, one per thread,
// held in registers; a 4 x 8-bit radix select finds the k-th key.
template <int MODE>
__global__ __launch_bounds__(IT) void index_merge_kernel(IndexPlan p) {
    extern __shared__ uint32_t dyn[];
    __shared__ IdxSmem sm;
    const int q = blockIdx.x, tid = threadIdx.x;
    const int b = q / p.Tq;
    uint32_t *pre = dyn;                                  // [n_chunks + 1] candidate offsets
    uint32_t *skey = dyn + p.n_chunks + 1;                // [chunk] (exact fallback)
    float *sq = (float *)(skey + p.chunk);                // f32 mode query
    if (MODE == 0) {
        const float *iq = (const float *)p.iq + (size_t)q * p.H * p.dI;
        for (int i = tid; i < p.H * p.dI; i += IT) sq[i] = iq[i];
    }
    const int64_t nvis = visible_entries(p, q);
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
    const uint32_t *meta = p.meta + (size_t)q * p.n_chunks * 2;
    // exclusive prefix of candidate counts over chunks
    int bad = 0;
    uint32_t carry = 0;
    for (int c0 = 0; c0 < p.n_chunks; c0 += IT) {
        const int c = c0 + tid;
        uint32_t n = c < p.n_chunks ? meta[2 * c] : 0u;
        if (n == 0xFFFFFFFFu) {
            bad = 1;
            n = 0;
        }
        uint32_t tot;
        const uint32_t inc = block_scan(n, sm, &tot);
        if (c < p.n_chunks) pre[c] = carry + inc - n;
        carry += tot;
        __syncthreads();
    }
    if (tid == 0) pre[p.n_chunks] = carry;
    const uint32_t total = carry;
    const uint32_t per = (total + IT - 1) / IT;
    __syncthreads();
    if (__syncthreads_or(bad) || per > REG_CAND) {
        exact_fallback<MODE>(p, q, b, nvis, kk, skey, sq, sm);
        return;
    }
    uint32_t keys[REG_CAND];
    int32_t ids[REG_CAND];
    int mine;
    if (p.n_chunks <= IT && __syncthreads_and(tid >= p.n_chunks || pre[tid + 1] - pre[tid] <= REG_CAND)) {
        // one chunk per thread: its whole region, in order
        mine = tid < p.n_chunks ? (int)(pre[tid + 1] - pre[tid]) : 0;
        const size_t base = ((size_t)q * p.n_chunks + tid) * p.region_cap;
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            keys[i] = i < mine ? p.reg_key[base + i] : 0u;
            ids[i] = i < mine ? p.reg_idx[base + i] : -1;
        }
    } else {
        // equal contiguous runs [lo, hi) of the flattened candidate list
        const uint32_t lo = min(total, tid * per), hi = min(total, lo + per);
        int c = 0;
        {
            int l = 0, r = p.n_chunks;  // last chunk with pre[c] <= lo
            while (r - l > 1) {
                const int mid = (l + r) >> 1;
                if (pre[mid] <= lo) l = mid;
                else r = mid;
            }
            c = l;
        }
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            keys[i] = 0u;
            ids[i] = -1;
            const uint32_t f = lo + i;
            if (f < hi) {
                while (pre[c + 1] <= f) ++c;
                const size_t slot = ((size_t)q * p.n_chunks + c) * p.region_cap + (f - pre[c]);
                keys[i] = p.reg_key[slot];
                ids[i] = p.reg_idx[slot];
            }
        }
        mine = (int)(hi - lo);
    }
    // radix select of the kk-th largest key
    uint32_t prefix = 0, mask = 0, need = (uint32_t)kk;
    for (int d = 3; d >= 0; --d) {
        for (int i = tid; i < 256; i += IT) sm.hist[i] = 0;
        __syncthreads();
        const int sh = 8 * d;
        // runs of equal bins are counted in a register first: the candidates
        // cluster in few bins, and same-address LDS atomics serialise
        uint32_t run_bin = 0xFFFFFFFFu, run = 0;
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            if (i < mine && (keys[i] & mask) == prefix) {
                const uint32_t bin = (keys[i] >> sh) & 255u;
                if (bin != run_bin) {
                    if (run) atomicAdd(&sm.hist[run_bin], run);
                    run_bin = bin;
                    run = 0;
                }
                ++run;
            }
        }
        if (run) atomicAdd(&sm.hist[run_bin], run);
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
    for (int cc = tid; cc < p.n_chunks; cc += IT) sat |= meta[2 * cc + 1] > kth;
    if (__syncthreads_or(sat)) {
        exact_fallback<MODE>(p, q, b, nvis, kk, skey, sq, sm);
        return;
    }
    // keys > kth, and the first `need` keys == kth in id order
    uint32_t nt = 0, ngt = 0;
#pragma unroll
    for (int i = 0; i < REG_CAND; ++i) {
        nt += (i < mine) && keys[i] == kth;
        ngt += (i < mine) && keys[i] > kth;
    }
    uint32_t tot;
    uint32_t tb = block_scan(nt, sm, &tot) - nt;
    const uint32_t ntake = ngt + (tb < need ? min(nt, need - tb) : 0u);
    uint32_t pos = block_scan(ntake, sm, &tot) - ntake;
#pragma unroll
    for (int i = 0; i < REG_CAND; ++i) {
        if (i < mine) {
            bool take = keys[i] > kth;
            if (keys[i] == kth) take = (tb++ < need);
            if (take) {
                oidx[pos] = ids[i];
                if (osc) osc[pos] = key_score(keys[i]);
                ++pos;
            }
        }
    }
    for (int i = kk + tid; i < p.k; i += IT) {
        oidx[i] = -1;
        if (osc) osc[i] = 0.f;
    }
}

template <int MODE>
static void launch_mode(const IndexPlan &p, hipStream_t s) {
    const size_t q_lds = MODE == 0 ? (size_t)p.H * p.dI * 4 : 0;
    hipLaunchKernelGGL(index_score_kernel<MODE>, dim3(p.n_chunks, p.Q), dim3(IT), (size_t)p.chunk * 4 + q_lds, s, p);
    hipLaunchKernelGGL(index_merge_kernel<MODE>, dim3(p.Q), dim3(IT),
                       (size_t)(p.n_chunks + 1 + p.chunk) * 4 + q_lds, s, p);
}

hipError_t launch_index(const IndexPlan &p, hipStream_t s) {
    if (p.keys.fmt == 0) launch_mode<0>(p, s);
    else switch (p.H / 16) {
            case 1: launch_mode<1>(p, s); break;
            case 2: launch_mode<2>(p, s); break;
            case 3: launch_mode<3>(p, s); break;
            default: launch_mode<4>(p, s); break;
        }
    return hipGetLastError();
}

}  // namespace v4a
