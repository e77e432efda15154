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
//  2. The chunk keeps its local top-s candidates: an LDS radix histogram of
//     11-bit digits of the order-preserving score key, taken from the highest
//     bit in which the chunk's keys differ and refined only while too many
//     entries reach the chosen bin, finds a threshold; every entry at or above
//     it is written, in index order, to the chunk's candidate region with the
//     threshold as the region's lower bound.
//  3. A merge kernel (one workgroup per query) radix-selects the k-th key over
//     the candidates held in registers, checks that no chunk could have
//     withheld an entry at or above it (lower bound > k-th key), and writes the
//     selection in ascending id order. If a chunk could have withheld one
//     (clustered winners, huge ties, region overflow) the merge falls back to
//     an exact radix select that rescores every visible entry.

#include "common.hpp"

namespace v4a {

constexpr int IT = 256;   // threads of a scoring workgroup (4 waves)
constexpr int MT = 1024;  // threads of the largest merge workgroup (16 waves)

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

struct IdxSmem {
    uint32_t hist[256];
    uint32_t scan[MT / 64 + 1];
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

// Values that are the same in every lane (the wave's index, an LDS word that
// every lane reads) are read into scalars, so that selections and loops on
// them are scalar compares and branches instead of per-lane masks.
__device__ __forceinline__ int wave_index() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }
__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// Per-wave values arr[0 .. NW) in LDS (NW <= 16): the sum over the waves
// before `wave` and over all of them, as scalars. Lane w < NW reads arr[w];
// a 16-lane inclusive scan (DPP row shifts) leaves the prefix sums in lanes
// 0 .. NW-1, which are read out with readlane.
template <int NW>
__device__ __forceinline__ void wave_prefix(const uint32_t *arr, int wave, uint32_t *before, uint32_t *all) {
    static_assert(NW >= 1 && NW <= 16, "the per-wave values fit one 16-lane row");
    const int lane = threadIdx.x & 63;
    uint32_t x = arr[lane < NW ? lane : 0];
    x = lane < NW ? x : 0u;
    if (NW > 1) x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
    if (NW > 2) x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
    if (NW > 4) x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
    if (NW > 8) x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
    *all = (uint32_t)__builtin_amdgcn_readlane((int)x, NW - 1);
    *before = wave > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)x, wave - 1) : 0u;
}

// Unsigned max of arr[0 .. NW) in LDS (NW <= 64), as a scalar.
template <int NW>
__device__ __forceinline__ uint32_t lds_max_u32(const uint32_t *arr) {
    const int lane = threadIdx.x & 63;
    return uniform_u32(wave_max_u32(arr[lane < NW ? lane : 0]));
}

// Inclusive prefix sum over the workgroup (NT threads) in thread order; *total gets the sum.
template <int NT>
__device__ uint32_t block_scan(uint32_t v, IdxSmem &sm, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = wave_index();
    const uint32_t x = wave_inclusive_scan(v);
    __syncthreads();
    if (lane == 63) sm.scan[wave] = x;
    __syncthreads();
    uint32_t before, all;
    wave_prefix<NT / 64>(sm.scan, wave, &before, &all);
    *total = all;
    return x + before;
}

// Largest bin b with sum(hist[b..255]) >= need. Returns b; *above = sum(hist[b+1..255]).
template <int NT>
__device__ int find_bin(IdxSmem &sm, uint32_t need, uint32_t *above) {
    const int tid = threadIdx.x;
    const uint32_t h = tid < 256 ? sm.hist[255 - tid] : 0u;  // thread t: bin 255-t
    uint32_t total;
    uint32_t suf = block_scan<NT>(h, sm, &total);
    uint32_t excl = suf - h;
    __syncthreads();
    if (tid < 256 && suf >= need && excl < need) {
        sm.misc[0] = 255 - tid;
        sm.misc[1] = (int)excl;
    }
    __syncthreads();
    int b = (int)uniform_u32((uint32_t)sm.misc[0]);
    *above = uniform_u32((uint32_t)sm.misc[1]);
    __syncthreads();
    return b;
}

// ------------------------------------------------------------- scoring ----

// Reduce-scatter over the four 16-lane rows: row g of the result holds, in
// each column, the sum over all four rows of x[g] (on the VALU, with the
// gfx950 lane-swap instructions). A 32-lane swap adds rows g and g + 2 of
// x[0] / x[2] and of x[1] / x[3]; a 16-lane swap then adds rows 2j and 2j + 1.
__device__ __forceinline__ float swap_add32(float a, float b) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float scatter_rows(const float (&x)[4]) {
    const float x02 = swap_add32(x[0], x[2]);  // rows 0, 1: x[0]; rows 2, 3: x[2] (two rows summed)
    const float x13 = swap_add32(x[1], x[3]);
    return swap_add16(x02, x13);               // row g: x[g] summed over the four rows
}


// max(0, d) propagating NaN (the IEEE 754-2019 maximum): a NaN dot product
// makes the entry's score NaN, which ranks below every number.
__device__ __forceinline__ float relu_nan(float d) { return (d > 0.0f || d != d) ? d : 0.0f; }

// sum_h w_h max(0, d_h) over this lane's heads, as an fma chain. The exact
// form is relu_nan. The fast form takes the max of the bit patterns as signed
// integers: one instruction, equal to the exact form for every d that is not
// NaN (a negative value or -0 gives +0, and +0 or -0 added to a chain that
// starts at +0 leaves it unchanged); the caller sends a tile to it only when
// the scale bytes rule out a NaN d.
template <int NT, bool FAST>
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
        for (int j = 0; j < 4; ++j) {
            const float r = FAST ? __int_as_float(__builtin_elementwise_max(__float_as_int(acc[i][j]), 0))
                                 : relu_nan(acc[i][j]);
            s = __builtin_fmaf(wv[i][j], r, s);
        }
    return s;
}

// Scores of entries [c0, c0+cnt) -> skey[0..IDX_CHUNK) (order-preserving
// keys; slots at or past cnt hold the score of an all-zero key and are never
// read). Wave w takes tiles w, w+NW, w+2NW, ... of 16 keys; a batch is four
// of them, one per 16-lane row, and two batches are in flight. Each lane
// loads one 16-byte quarter of one key row per tile through a buffer
// resource that ends at the chunk's last row, so loads past the end return
// zeros with no address clamping and no branch. After the per-lane head sums
// of a batch, one reduce-scatter over the rows leaves lane (row g, column c)
// with the score of key c of the batch's tile g: one score key and one LDS
// store per lane per batch.
template <int NT, bool FASTOK>
__device__ void score_chunk_mx(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey) {
    constexpr int NW = IT / 64, BATCH = 4;
    constexpr int STRIDE = NW * BATCH;               // tiles per batch over the NW waves
    constexpr int NB = IDX_CHUNK / (16 * STRIDE);    // batches per wave
    constexpr int DEPTH = 3;                         // batches in flight per wave
    static_assert(NB * 16 * STRIDE == IDX_CHUNK && NB >= DEPTH, "a chunk is at least DEPTH batches");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 15, grp = lane >> 4;

    // Issue order: the query's raw operands, then the first DEPTH key batches;
    // the query is first used after they are all issued. The memory clobbers
    // pin that order in the IR, the scheduling barriers in the machine
    // scheduler, and the register fences keep every use of the query values
    // (even their unpacking) behind the key loads.
    const uint8_t *iq = (const uint8_t *)p.iq + (size_t)q * p.H * 64;
    const uint8_t *iqs = p.iq_scale + (size_t)q * p.H * 4;
    const float *w = p.w + (size_t)q * p.H;
    v4i qv[4];
    uint32_t qsc[4];
    float wv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qv[i] = (v4i){0, 0, 0, 0};
        qsc[i] = 0;
        if (i < NT) {
            qv[i] = *(const v4i *)(iq + (16 * i + col) * 64 + 16 * grp);
            qsc[i] = iqs[(16 * i + col) * 4 + grp];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[i][j] = (i < NT) ? w[16 * i + 4 * grp + j] : 0.f;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    const char *kbase = p.keys.e2m1 + (int64_t)b * p.keys.e2m1_bs + c0 * p.keys.e2m1_rs;
    const char *sbase = p.keys.e8m0 + (int64_t)b * p.keys.e8m0_bs + c0 * p.keys.e8m0_rs;
    const uint32_t krs = (uint32_t)p.keys.e2m1_rs, srs = (uint32_t)p.keys.e8m0_rs;
    // byte ranges of the chunk's rows: the last row ends at (cnt - 1) * stride + row bytes
    const uint32_t kbytes = (uint32_t)(cnt - 1) * krs + 64u, sbytes = (uint32_t)(cnt - 1) * srs + 4u;
    const uint32_t kvo = (uint32_t)(wave * 16 + col) * krs + 16u * grp;  // this lane's quarter in tile `wave`
    const uint32_t svo = (uint32_t)(wave * 16 + col) * srs;              // the row's four exponents (one word)
    v4i kbuf[DEPTH][BATCH];
    uint32_t sbuf[DEPTH][BATCH];
    auto issue = [&](v4i (&kv)[BATCH], uint32_t (&sv)[BATCH], int bi) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            // the tile's offset is uniform: it moves the resource base (scalar work only)
            const uint32_t t16 = (uint32_t)(STRIDE * bi + NW * u) * 16u;
            const uint32_t ko = t16 * krs, so = t16 * srs;
            const int nk = (int)kbytes - (int)ko, ns = (int)sbytes - (int)so;  // bytes left (max on the SALU)
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(kbase + ko), (short)0, __builtin_elementwise_max(nk, 0), 0x00020000);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(sbase + so), (short)0, __builtin_elementwise_max(ns, 0), 0x00020000);
            kv[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, kvo, 0, 2);  // nontemporal
            sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, svo, 0, 2);
        }
    };
    // each batch (keys and exponents) wholly ahead of the next
#pragma unroll
    for (int i = 0; i < DEPTH; ++i) {
        issue(kbuf[i], sbuf[i], i);
        __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        asm volatile("" : "+v"(qv[i]), "+v"(qsc[i]));
#pragma unroll
        for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(wv[i][j]));
    }

    v8i A[4];
    uint32_t sA = 0, qmax = 0, qnan = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        A[i] = (v8i){qv[i][0], qv[i][1], qv[i][2], qv[i][3], 0, 0, 0, 0};
        sA |= qsc[i] << (8 * i);
        qmax = qsc[i] > qmax ? qsc[i] : qmax;
        qnan |= qsc[i] == 0xFFu;
    }
    // A tile takes the fast form when no d can be NaN: no scale byte is 0xFF
    // (NaN) and nothing overflows. Each of the 128 products is at most
    // 6 * 6 * 2^(ea - 127) * 2^(eb - 127) for block exponent bytes ea, eb, so
    // |d| and every partial sum stay below 2^(12.2 + ea + eb - 254), finite
    // while ea + eb <= 369. Hence: every key byte of the tile below
    // lim = min(370 - max query byte, 255); a NaN query scale sends every tile
    // to the exact form.
    qmax = wave_max_u32(qmax);
    const bool q_nan = __ballot(qnan != 0) != 0;
    int lim = 370 - (int)qmax;
    lim = lim > 255 ? 255 : lim;
    if (q_nan || !FASTOK) lim = 0;

    auto unpack = [&](uint32_t (&sv)[BATCH]) {
        // the fence keeps every use of the batch (even the byte extraction) behind the previous issue
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            asm volatile("" : "+v"(sv[u]));
            sv[u] = (sv[u] >> (8 * grp)) & 0xFFu;  // this lane's K block: exponent byte grp
        }
    };
    auto finish = [&](const float (&part)[BATCH], int bi) {
        const float s = scatter_rows(part);
        skey[(STRIDE * bi + wave + NW * grp) * 16 + col] = score_key(s);
    };
    // fast pass: every tile in the fast form; a batch with a key byte at or
    // above lim only marks the wave for the exact pass below
    bool redo = !FASTOK || q_nan;
    auto consume = [&](const v4i (&kv)[BATCH], uint32_t (&sv)[BATCH], int bi) {
        unpack(sv);
        const uint32_t smax = __builtin_elementwise_max(__builtin_elementwise_max(sv[0], sv[1]),
                                                        __builtin_elementwise_max(sv[2], sv[3]));
        redo |= __ballot((int)smax >= lim) != 0;
        float part[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) part[u] = head_sum<NT, true>(A, sA, kv[u], sv[u], wv);
        finish(part, bi);
    };
    if (FASTOK) {
        // DEPTH batches in flight: batch bi + DEPTH is issued into the registers
        // of batch bi as soon as bi is consumed (scheduling barriers around each
        // issue keep the next batch's work from being hoisted above it, which
        // would wait for that batch's data first)
#pragma unroll
        for (int bi = 0; bi < NB; ++bi) {
            consume(kbuf[bi % DEPTH], sbuf[bi % DEPTH], bi);
            __builtin_amdgcn_sched_barrier(0);
            if (bi + DEPTH < NB) issue(kbuf[bi % DEPTH], sbuf[bi % DEPTH], bi + DEPTH);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // exact pass (rare: extreme exponents, NaN scales, or the merge's exact
    // select): the wave rescores its own tiles one batch at a time, in a
    // separate loop so that its registers never add to the fast pass's
    if (redo) {
        for (int bi = 0; bi < NB; ++bi) {
            issue(kbuf[0], sbuf[0], bi);
            unpack(sbuf[0]);
            float part[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) part[u] = head_sum<NT, false>(A, sA, kbuf[0][u], sbuf[0][u], wv);
            finish(part, bi);
        }
    }
}

constexpr int F32_MAX_H = 16;

// float32 keys: one entry per thread, dot products in float64.
template <int NTH>
__device__ void score_chunk_f32(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey,
                                const float *sq) {
    const int H = p.H, dI = p.dI;
    const float *w = p.w + (size_t)q * H;
    for (int r = threadIdx.x; r < cnt; r += NTH) {
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
            if (h < H) s += (double)w[h] * ((acc[h] > 0.0 || acc[h] != acc[h]) ? acc[h] : 0.0);
        skey[r] = score_key((float)s);
    }
}

// MODE 0: f32 keys, 1..4: MXFP4 with MODE head tiles (IT threads); NTH
// threads for the f32 form; FASTOK: tiles may take the fast ReLU form
template <int MODE, int NTH, bool FASTOK = true>
__device__ __forceinline__ void score_chunk(const IndexPlan &p, int q, int b, int64_t c0, int cnt, uint32_t *skey,
                                            const float *sq) {
    if (MODE == 0) score_chunk_f32<NTH>(p, q, b, c0, cnt, skey, sq);
    else score_chunk_mx<MODE, FASTOK>(p, q, b, c0, cnt, skey);
}

// ---------------------------------------------------- chunk candidates ----

// Keep the chunk's entries at or above a threshold that at least s of them
// reach. The threshold is the lower edge of a radix bin: 11-bit digits taken
// from the highest bit in which the chunk's keys differ, so the bins follow
// the keys' actual range; the bin holding the s-th largest key is refined by
// further digits only while the entries at or above its edge are more than a
// merge thread group takes in registers (EMIT_SOFT), or than twice s where s
// exceeds that. Entries are written in index order with the threshold as the
// region's lower bound.
constexpr int EBITS = 11;
constexpr int EBINS = 1 << EBITS;
constexpr int EMIT_SOFT = 32;  // = merge_group * merge_rc of the merge (static_assert there)
struct EmitSmem {
    uint32_t hist[EBINS] __attribute__((aligned(16)));
    uint32_t red[2][IT / 64];
    uint32_t scan[IT / 64];
    uint32_t res[4];
};

// Exclusive prefix sum over the IT threads in thread order; *total gets the sum.
__device__ __forceinline__ uint32_t emit_scan(uint32_t v, EmitSmem &em, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = wave_index();
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) em.scan[wave] = x;
    __syncthreads();
    uint32_t before, all;
    wave_prefix<IT / 64>(em.scan, wave, &before, &all);
    *total = all;
    return x - v + before;
}

// PER: entries per thread, in index order (the chunk holds IT x PER).
// FULL: the chunk holds IT * PER entries (every slot valid).
template <int PER, bool FULL>
__device__ void chunk_emit_impl(const IndexPlan &p, int q, int chunk, int64_t c0, int cnt, int s_want,
                                const uint32_t *skey, EmitSmem &em) {
    static_assert(PER % 4 == 0, "whole 16-byte LDS reads per thread");
    const int tid = threadIdx.x, lane = tid & 63, wave = wave_index();
    const size_t rid = (size_t)q * p.n_chunks + chunk;
    uint32_t key[PER];
#pragma unroll
    for (int v = 0; v < PER / 4; ++v) {
        const uint4 k4 = *(const uint4 *)&skey[PER * tid + 4 * v];
        key[4 * v] = k4.x;
        key[4 * v + 1] = k4.y;
        key[4 * v + 2] = k4.z;
        key[4 * v + 3] = k4.w;
    }
    bool valid[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) valid[j] = FULL || PER * tid + j < cnt;
    uint32_t thr = 0;  // emit valid keys >= thr
    if (cnt > s_want) {
        // range of the valid keys; the histogram is cleared in the same round
        uint32_t mx = 0u, mn = 0xFFFFFFFFu;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            mx = __builtin_elementwise_max(mx, valid[j] ? key[j] : 0u);
            mn = __builtin_elementwise_min(mn, valid[j] ? key[j] : 0xFFFFFFFFu);
        }
        mx = wave_max_u32(mx);
        uint32_t nmn = wave_max_u32(~mn);
        *(uint4 *)&em.hist[8 * tid] = make_uint4(0, 0, 0, 0);
        *(uint4 *)&em.hist[8 * tid + 4] = make_uint4(0, 0, 0, 0);
        if (lane == 0) {
            em.red[0][wave] = mx;
            em.red[1][wave] = nmn;
        }
        __syncthreads();
        mx = lds_max_u32<IT / 64>(em.red[0]);
        nmn = lds_max_u32<IT / 64>(em.red[1]);
        const uint32_t diff = mx ^ ~nmn;
        if (diff == 0u) {
            thr = mx;  // every valid key equal: all of them reach it
        } else {
            // refine while more than `soft` would be emitted: EMIT_SOFT (what a
            // merge thread group takes) or, where every chunk must emit more than
            // that anyway (many chunks per query: chunked prefill), twice the
            // share; never more than the region holds
            uint32_t soft = 2u * (uint32_t)s_want > (uint32_t)EMIT_SOFT ? 2u * (uint32_t)s_want : (uint32_t)EMIT_SOFT;
            soft = soft < (uint32_t)p.region_cap ? soft : (uint32_t)p.region_cap;
            int top = 31 - __builtin_clz(diff);  // highest differing bit; bits above it are common
            uint32_t prefix = (uint32_t)(((uint64_t)mx >> (top + 1)) << (top + 1));
            uint32_t need = (uint32_t)s_want, above_all = 0;
            bool refining = false;  // the first digit: every valid key shares the bits above top
            while (true) {
                const int sh = top + 1 - EBITS > 0 ? top + 1 - EBITS : 0;
                const uint32_t dmask = (2u << (top - sh)) - 1u;
                if (!refining) {
#pragma unroll
                    for (int j = 0; j < PER; ++j)
                        if (valid[j]) atomicAdd(&em.hist[(key[j] >> sh) & dmask], 1u);
                } else {
#pragma unroll
                    for (int j = 0; j < PER; ++j)
                        if (valid[j] && ((uint64_t)key[j] >> (top + 1)) == ((uint64_t)prefix >> (top + 1)))
                            atomicAdd(&em.hist[(key[j] >> sh) & dmask], 1u);
                }
                __syncthreads();
                // thread t owns bins EBINS-8(t+1) .. EBINS-8t-1, highest first
                const uint4 h1 = *(const uint4 *)&em.hist[EBINS - 8 * tid - 4];
                const uint4 h0 = *(const uint4 *)&em.hist[EBINS - 8 * tid - 8];
                const uint32_t h[8] = {h1.w, h1.z, h1.y, h1.x, h0.w, h0.z, h0.y, h0.x};
                uint32_t local = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) local += h[i];
                uint32_t tot;
                const uint32_t before = emit_scan(local, em, &tot);
                if (before < need && need <= before + local) {
                    uint32_t c = before;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        if (c < need && need <= c + h[i]) {
                            em.res[0] = EBINS - 1 - 8 * tid - i;
                            em.res[1] = c;     // keys in higher bins
                            em.res[2] = h[i];  // keys in the bin
                        }
                        c += h[i];
                    }
                }
                __syncthreads();
                const uint32_t bin = uniform_u32(em.res[0]), above = uniform_u32(em.res[1]),
                               pop = uniform_u32(em.res[2]);
                prefix |= bin << sh;
                above_all += above;
                need -= above;
                if (above_all + pop <= soft || sh == 0) break;
                // refine inside the bin: clear it for the next digit
                __syncthreads();  // every thread has read res and its bins
                *(uint4 *)&em.hist[8 * tid] = make_uint4(0, 0, 0, 0);
                *(uint4 *)&em.hist[8 * tid + 4] = make_uint4(0, 0, 0, 0);
                __syncthreads();
                top = sh - 1;
                refining = true;
            }
            thr = prefix;
        }
    }
    // compaction in index order
    uint32_t mine = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) mine += (valid[j] && key[j] >= thr) ? 1u : 0u;
    uint32_t total;
    uint32_t off = emit_scan(mine, em, &total);
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
#pragma unroll
    for (int j = 0; j < PER; ++j) {
        if (valid[j] && key[j] >= thr) {
            rk[off] = key[j];
            ri[off] = (int32_t)(c0 + PER * tid + j);
            ++off;
        }
    }
    if (tid == 0) {
        meta[0] = total;
        meta[1] = thr;
    }
}

template <int PER>
__device__ __forceinline__ void chunk_emit(const IndexPlan &p, int q, int chunk, int64_t c0, int cnt, int s_want,
                                           const uint32_t *skey, EmitSmem &em) {
    if (cnt == IT * PER) chunk_emit_impl<PER, true>(p, q, chunk, c0, cnt, s_want, skey, em);
    else chunk_emit_impl<PER, false>(p, q, chunk, c0, cnt, s_want, skey, em);
}

// ------------------------------------------------------------- merge ----

// The merge workgroup holds MERGE_SLOTS candidates in registers: NT threads
// of merge_rc<NT>() each, merge_group<NT>() threads sharing one chunk's region.
constexpr int MERGE_SLOTS = 8192;
constexpr int MERGE_WIDE_Q = 512;  // from this many queries per call the merge takes 512 threads per query
template <int NT> constexpr int merge_rc() { return MERGE_SLOTS / NT; }
template <int NT> constexpr int merge_group() { return EMIT_SOFT / merge_rc<NT>(); }
static_assert(merge_group<1024>() * merge_rc<1024>() == EMIT_SOFT && merge_group<512>() * merge_rc<512>() == EMIT_SOFT,
              "a chunk emits at most what one thread group holds");

template <int MODE, int NT>
__device__ void exact_fallback(const IndexPlan &p, int q, int b, int64_t nvis, int kk, uint32_t *skey,
                               const float *sq, IdxSmem &sm) {
    // Radix select over every visible entry, rescoring chunk by chunk.
    const int tid = threadIdx.x;
    uint32_t prefix = 0, mask = 0, need = (uint32_t)kk;
    for (int d = 3; d >= 0; --d) {
        for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
        __syncthreads();
        for (int64_t c0 = 0; c0 < nvis; c0 += IDX_CHUNK) {
            const int cnt = (int)((nvis - c0) < IDX_CHUNK ? (nvis - c0) : IDX_CHUNK);
            if (threadIdx.x < IT) score_chunk<MODE, IT, false>(p, q, b, c0, cnt, skey, sq);  // the first IT threads score
            __syncthreads();
            for (int i = tid; i < cnt; i += NT)
                if ((skey[i] & mask) == prefix) atomicAdd(&sm.hist[(skey[i] >> (8 * d)) & 255u], 1u);
            __syncthreads();
        }
        uint32_t above;
        const int bin = find_bin<NT>(sm, need, &above);
        need -= above;
        prefix |= (uint32_t)bin << (8 * d);
        mask |= 255u << (8 * d);
    }
    // kth key = prefix; take every key > prefix and the first `need` equal ones.
    int32_t *oidx = p.out_idx + (size_t)q * p.k;
    float *osc = p.out_score ? p.out_score + (size_t)q * p.k : nullptr;
    uint32_t written = 0, ties = 0;
    const int per = (IDX_CHUNK + NT - 1) / NT;
    for (int64_t c0 = 0; c0 < nvis; c0 += IDX_CHUNK) {
        const int cnt = (int)((nvis - c0) < IDX_CHUNK ? (nvis - c0) : IDX_CHUNK);
        if (threadIdx.x < IT) score_chunk<MODE, IT, false>(p, q, b, c0, cnt, skey, sq);  // the first IT threads score
        __syncthreads();
        const int lo = threadIdx.x * per;
        uint32_t nt = 0;
        for (int i = lo; i < lo + per && i < cnt; ++i) nt += skey[i] == prefix;
        uint32_t tot_t;
        uint32_t tie_before = ties + block_scan<NT>(nt, sm, &tot_t) - nt;
        uint32_t ns = 0;
        {
            uint32_t tb = tie_before;
            for (int i = lo; i < lo + per && i < cnt; ++i) {
                if (skey[i] > prefix) ++ns;
                else if (skey[i] == prefix) ns += (tb++ < need);
            }
        }
        uint32_t tot_s;
        uint32_t pos = written + block_scan<NT>(ns, sm, &tot_s) - ns;
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
    for (int i = kk + tid; i < p.k; i += NT) {
        oidx[i] = -1;
        if (osc) osc[i] = 0.f;
    }
}

// ------------------------------------------------------------ kernels ----

template <int MODE>
__global__ __launch_bounds__(IT) void index_score_kernel(IndexPlan p) {
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ EmitSmem em;
    uint32_t *skey = dyn;                                 // [chunk]
    float *sq = (float *)(dyn + p.chunk);                 // f32 mode: query [H][dI]
    const int chunk = blockIdx.x, q = blockIdx.y + p.q_base;
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
    score_chunk<MODE, IT>(p, q, b, c0, cnt, skey, sq);
    __syncthreads();
    // every full chunk keeps enough that the union holds at least kk entries
    const int64_t n_active = (nvis + p.chunk - 1) / p.chunk;
    int s_want = p.s_local;
    const int64_t div = n_active > 1 ? n_active - 1 : 1;
    const int64_t spread = (kk + div - 1) / div;
    if (spread > s_want) s_want = (int)spread;
    if (s_want > cnt) s_want = cnt;
    chunk_emit<IDX_CHUNK / IT>(p, q, chunk, c0, cnt, s_want, skey, em);
}

// ---------------------------------------- several chunks per workgroup ----

// Several queries per sequence over many entries (chunked prefill, drafts).
// A chunk is IDX_CPW sub-chunks of IDX_CHUNK entries; the workgroup of
// (chunk, query) loads the query's operands once, scores the sub-chunks one
// after the other (the next one's first two key batches in flight while the
// current one finishes) into one score buffer, and emits the chunk's
// candidates once. Per sub-chunk the tiles, head sums and score keys are
// those of score_chunk_mx, so every score is bitwise the one-chunk kernel's.
// One emission per IDX_CPW sub-chunks: the emission's fixed VALU work, and
// not the head sums, was what an emission per sub-chunk spent beyond them.

struct ChunkGeo {
    const char *kbase, *sbase;
    uint32_t kbytes, sbytes;  // byte ranges of the chunk's visible rows
};

__device__ __forceinline__ ChunkGeo chunk_geo(const IndexPlan &p, int b, int64_t c0, int cnt) {
    ChunkGeo g;
    g.kbase = p.keys.e2m1 + (int64_t)b * p.keys.e2m1_bs + c0 * p.keys.e2m1_rs;
    g.sbase = p.keys.e8m0 + (int64_t)b * p.keys.e8m0_bs + c0 * p.keys.e8m0_rs;
    g.kbytes = (uint32_t)(cnt - 1) * (uint32_t)p.keys.e2m1_rs + 64u;
    g.sbytes = (uint32_t)(cnt - 1) * (uint32_t)p.keys.e8m0_rs + 4u;
    return g;
}

template <int NT>
__global__ __launch_bounds__(IT, 4) void index_score_cpw_kernel(IndexPlan p) {
    constexpr int NW = IT / 64, BATCH = 4;
    constexpr int STRIDE = NW * BATCH;
    constexpr int NB = IDX_CHUNK / (16 * STRIDE);
    static_assert(NB * 16 * STRIDE == IDX_CHUNK && NB % 2 == 0, "a chunk is an even number of batches");
    extern __shared__ __attribute__((aligned(16))) uint32_t dyn[];
    __shared__ EmitSmem em;
    uint32_t *skey = dyn;  // [chunk]: sub-chunk i's scores from IDX_CHUNK i on
    const int q = blockIdx.y + p.q_base;
    const int b = q / p.Tq;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int chunk = blockIdx.x;
    const int64_t cbase = (int64_t)chunk * p.chunk;
    const int64_t nvis = visible_entries(p, q);
    const int64_t n_active = (nvis + p.chunk - 1) / p.chunk;
    const int cnt_all = (int)(nvis - cbase <= 0 ? 0 : (nvis - cbase < p.chunk ? nvis - cbase : p.chunk));
    if (cnt_all == 0) {
        if (tid == 0) {
            uint32_t *meta = p.meta + ((size_t)q * p.n_chunks + chunk) * 2;
            meta[0] = 0;
            meta[1] = 0;
        }
        return;
    }
    const int n_sub = (cnt_all + IDX_CHUNK - 1) / IDX_CHUNK;  // sub-chunks with visible entries

    // the query's operands into LDS (read again for each chunk, so that they
    // hold no registers while the next chunk's keys fly during an emission)
    constexpr int H = 16 * NT;
    uint8_t *s_iq = (uint8_t *)(dyn + p.chunk);  // [H][64]
    uint8_t *s_iqs = s_iq + H * 64;              // [H][4]
    float *s_w = (float *)(s_iqs + H * 4);       // [H]
    {
        const uint8_t *iq = (const uint8_t *)p.iq + (size_t)q * H * 64;
        uint4 x = make_uint4(0, 0, 0, 0);
        uint32_t y = 0;
        float z = 0.f;
        if (tid < H * 4) {
            x = ((const uint4 *)iq)[tid];
            y = p.iq_scale[(size_t)q * H * 4 + tid];
        }
        if (tid < H) z = p.w[(size_t)q * H + tid];
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        if (tid < H * 4) {
            ((uint4 *)s_iq)[tid] = x;
            s_iqs[tid] = (uint8_t)y;
        }
        if (tid < H) s_w[tid] = z;
    }
    const uint32_t krs = (uint32_t)p.keys.e2m1_rs, srs = (uint32_t)p.keys.e8m0_rs;
    const uint32_t kvo = (uint32_t)(wave * 16 + col) * krs + 16u * grp;
    const uint32_t svo = (uint32_t)(wave * 16 + col) * srs;
    v4i ka[BATCH], kb[BATCH];
    uint32_t sa[BATCH], sb[BATCH];
    auto issue = [&](v4i (&kv)[BATCH], uint32_t (&sv)[BATCH], const ChunkGeo &g, int bi) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            const uint32_t t16 = (uint32_t)(STRIDE * bi + NW * u) * 16u;
            const uint32_t ko = t16 * krs, so = t16 * srs;
            const int nk = (int)g.kbytes - (int)ko, ns = (int)g.sbytes - (int)so;
            const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(g.kbase + ko), (short)0, __builtin_elementwise_max(nk, 0), 0x00020000);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void *)(g.sbase + so), (short)0, __builtin_elementwise_max(ns, 0), 0x00020000);
            kv[u] = __builtin_amdgcn_raw_buffer_load_b128(rk, kvo, 0, 0);
            sv[u] = __builtin_amdgcn_raw_buffer_load_b32(rs, svo, 0, 0);
        }
    };
    auto sub_cnt = [&](int sub) {
        const int left = cnt_all - sub * IDX_CHUNK;
        return left < IDX_CHUNK ? left : IDX_CHUNK;
    };
    ChunkGeo geo = chunk_geo(p, b, cbase, sub_cnt(0));
    issue(ka, sa, geo, 0);
    __builtin_amdgcn_sched_barrier(0);
    issue(kb, sb, geo, 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // the query is in LDS
    // the fast-form rule of score_chunk_mx (uniform over the workgroup's chunks)
    uint32_t sA = 0, qmax = 0, qnan = 0;
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const uint32_t sc = s_iqs[(16 * i + col) * 4 + grp];
        sA |= sc << (8 * i);
        qmax = sc > qmax ? sc : qmax;
        qnan |= sc == 0xFFu;
    }
    qmax = wave_max_u32(qmax);
    const bool q_nan = __ballot(qnan != 0) != 0;
    int lim = 370 - (int)qmax;
    lim = lim > 255 ? 255 : lim;
    if (q_nan) lim = 0;
    // every full chunk keeps enough that the union holds at least kk entries (as the one-chunk kernel)
    const int kk = (int)(nvis < p.k ? nvis : p.k);
    int s_base = p.s_local;
    {
        const int64_t div = n_active > 1 ? n_active - 1 : 1;
        const int64_t spread = (kk + div - 1) / div;
        if (spread > s_base) s_base = (int)spread;
    }

    auto unpack = [&](uint32_t (&sv)[BATCH]) {
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            asm volatile("" : "+v"(sv[u]));
            sv[u] = (sv[u] >> (8 * grp)) & 0xFFu;
        }
    };
    uint32_t *sk = skey;  // the current sub-chunk's scores
    auto finish = [&](const float (&part)[BATCH], int bi) {
        const float s = scatter_rows(part);
        sk[(STRIDE * bi + wave + NW * grp) * 16 + col] = score_key(s);
    };
    for (int sub = 0; sub < n_sub; ++sub) {
        sk = skey + sub * IDX_CHUNK;
        v8i A[4];
        float wv[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            A[i] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
            if (i < NT) {
                const v4i x = *(const v4i *)&s_iq[(16 * i + col) * 64 + 16 * grp];
                A[i] = (v8i){x[0], x[1], x[2], x[3], 0, 0, 0, 0};
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[i][j] = i < NT ? s_w[16 * i + 4 * grp + j] : 0.f;
        }
        bool redo = q_nan;
        auto consume = [&](const v4i (&kv)[BATCH], uint32_t (&sv)[BATCH], int bi) {
            unpack(sv);
            const uint32_t smax = __builtin_elementwise_max(__builtin_elementwise_max(sv[0], sv[1]),
                                                            __builtin_elementwise_max(sv[2], sv[3]));
            redo |= __ballot((int)smax >= lim) != 0;
            float part[BATCH];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) part[u] = head_sum<NT, true>(A, sA, kv[u], sv[u], wv);
            finish(part, bi);
        };
#pragma unroll
        for (int bi = 0; bi < NB; bi += 2) {
            consume(ka, sa, bi);
            __builtin_amdgcn_sched_barrier(0);
            if (bi + 2 < NB) issue(ka, sa, geo, bi + 2);
            __builtin_amdgcn_sched_barrier(0);
            consume(kb, sb, bi + 1);
            __builtin_amdgcn_sched_barrier(0);
            if (bi + 3 < NB) issue(kb, sb, geo, bi + 3);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (redo) {  // the exact pass of score_chunk_mx, over this wave's tiles
            for (int bi = 0; bi < NB; ++bi) {
                issue(ka, sa, geo, bi);
                unpack(sa);
                float part[BATCH];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) part[u] = head_sum<NT, false>(A, sA, ka[u], sa[u], wv);
                finish(part, bi);
            }
        }
        if (sub + 1 < n_sub) {  // the next sub-chunk's first batches
            geo = chunk_geo(p, b, cbase + (int64_t)(sub + 1) * IDX_CHUNK, sub_cnt(sub + 1));
            issue(ka, sa, geo, 0);
            __builtin_amdgcn_sched_barrier(0);
            issue(kb, sb, geo, 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    chunk_emit<IDX_CHUNK * IDX_CPW / IT>(p, q, chunk, cbase, cnt_all, s_base < cnt_all ? s_base : cnt_all, skey, em);
}

// ------------------------------------------------------ merge select ----

constexpr int MBITS = 12;                 // radix digit of the merge select
constexpr int MBINS = 1 << MBITS;
constexpr int RESOLVE_MAX = 128;          // a boundary bin this small is gathered and ranked directly
constexpr int STAGE_MAX = 2048;           // selections staged in LDS for coalesced output

// Per-key loops are kept free of branches: a key that does not count goes
// to a dummy slot of its lane (the arrays carry 64 extra slots).
template <int NT>
struct __attribute__((aligned(16))) MergeSmem {
    uint32_t hist[MBINS + 64];
    uint32_t part[2][NT / 64];  // wave totals of block scans (two buffers, used in turn)
    uint32_t red[3][NT / 64];
    uint32_t list[RESOLVE_MAX + 64] __attribute__((aligned(16)));
    uint32_t misc[4];
    uint32_t stage_key[STAGE_MAX + 64];  // selected keys, staged for coalesced output
};

// Inclusive prefix sum over the workgroup. Consecutive calls must alternate
// `buf`; the barrier of one call then protects the other buffer.
template <int NT>
__device__ __forceinline__ uint32_t scan_buf(uint32_t v, MergeSmem<NT> &sm, int buf, uint32_t *total) {
    const int lane = threadIdx.x & 63, wave = wave_index();
    const uint32_t x = wave_inclusive_scan(v);
    if (lane == 63) sm.part[buf][wave] = x;
    __syncthreads();
    uint32_t before, all;
    wave_prefix<NT / 64>(sm.part[buf], wave, &before, &all);
    *total = all;
    return x + before;
}

// Highest bin whose suffix count reaches `need`: its index, the count above
// it, its own count and the count over all bins. Thread t covers bins
// [MBINS - BPT(t+1), MBINS - BPT t) and zeroes them for the next pass.
template <int NT>
__device__ __forceinline__ void merge_find(MergeSmem<NT> &sm, uint32_t need, int buf, uint32_t *bin, uint32_t *above,
                                           uint32_t *in_bin, uint32_t *total) {
    constexpr int BPT = MBINS / NT;  // bins per thread, read as 16-byte words
    static_assert(BPT % 4 == 0, "whole 16-byte words of bins per thread");
    const int b0 = MBINS - BPT * (threadIdx.x + 1);
    uint32_t h[BPT];
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) {
        const uint4 x = *(const uint4 *)&sm.hist[b0 + 4 * v];
        h[4 * v] = x.x;
        h[4 * v + 1] = x.y;
        h[4 * v + 2] = x.z;
        h[4 * v + 3] = x.w;
    }
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < BPT; ++j) local += h[j];
    const uint32_t incl = scan_buf<NT>(local, sm, buf, total);
    uint32_t acc = incl - local;
    if (acc < need && incl >= need) {
#pragma unroll
        for (int j = BPT - 1; j >= 0; --j) {
            if (acc + h[j] >= need) {
                sm.misc[0] = (uint32_t)(b0 + j);
                sm.misc[1] = acc;
                sm.misc[2] = h[j];
                break;
            }
            acc += h[j];
        }
    }
#pragma unroll
    for (int v = 0; v < BPT / 4; ++v) *(uint4 *)&sm.hist[b0 + 4 * v] = make_uint4(0, 0, 0, 0);
    __syncthreads();
    *bin = uniform_u32(sm.misc[0]);
    *above = uniform_u32(sm.misc[1]);
    *in_bin = uniform_u32(sm.misc[2]);
}


// Marks the key registers as rewritten (no instruction is emitted), so that
// per-key tests are not hoisted out of the select loop into 32 live masks.
template <int RC>
__device__ __forceinline__ void fence_keys(uint32_t (&k)[RC]) {
#pragma unroll
    for (int i = 0; i < RC; ++i) asm volatile("" : "+v"(k[i]));
}

// One workgroup per query. Each thread holds a contiguous run of the chunks'
// candidates (in ascending id order) in registers: a quarter of its chunk's
// region when every chunk fits in 32 slots, else an equal share of the
// flattened list.
//
// Every chunk emitted all of its entries at or above its lower bound, so with
// T_lo = the largest lower bound, the candidates at or above T_lo are exactly
// the entries at or above T_lo. If at least k of them exist, the k-th key
// lies there and the candidates decide the selection exactly; otherwise the
// exact fallback runs. The k-th key is found by radix passes of MBITS-bit
// digits over [T_lo, max key], starting at the highest bit where the two
// differ; once the boundary bin holds at most RESOLVE_MAX keys they are
// gathered and ranked directly.
//
// Registers hold key + 1 (keys never reach 2^32 - 1: NaN maps to 0), so an
// empty slot is 0 and falls below every bound without a validity mask.
//
// merge_select is the candidate select; false when the exact fallback has to
// decide instead.
template <int NT>
__device__ __forceinline__ bool merge_select(const IndexPlan &p, int q, int kk, uint32_t *pre, IdxSmem &sm,
                                             MergeSmem<NT> &ms) {
    constexpr int REG_CAND = merge_rc<NT>(), GROUP = merge_group<NT>();
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = wave_index();
    int32_t *oidx = p.out_idx + (size_t)q * p.k;
    float *osc = p.out_score ? p.out_score + (size_t)q * p.k : nullptr;
    const uint32_t *meta = p.meta + (size_t)q * p.n_chunks * 2;
    if (tid == 0) ms.misc[3] = 0u;  // the gather's slot counter (read after later barriers)

    uint32_t keys[REG_CAND];
    int32_t ids[REG_CAND];
    int mine = 0;
    uint32_t t_lo = 1;  // largest chunk lower bound (+1) seen by this thread
    int over = 0, big = 1;
    if (p.n_chunks * GROUP <= NT) {
        // region mode: the region load is issued together with the count
        const int c = tid / GROUP, sub = tid % GROUP;
        uint32_t cnt = 0;
        if (c < p.n_chunks) {
            const uint2 mt = *(const uint2 *)(meta + 2 * c);
            cnt = mt.x;
            t_lo = mt.y + 1u;
            const size_t base = ((size_t)q * p.n_chunks + c) * p.region_cap + sub * REG_CAND;
            const uint4 *rk = (const uint4 *)(p.reg_key + base);
            const uint4 *ri = (const uint4 *)(p.reg_idx + base);
#pragma unroll
            for (int v = 0; v < REG_CAND / 4; ++v) {
                const uint4 kx = rk[v], ix = ri[v];
                keys[4 * v + 0] = kx.x; keys[4 * v + 1] = kx.y; keys[4 * v + 2] = kx.z; keys[4 * v + 3] = kx.w;
                ids[4 * v + 0] = (int32_t)ix.x; ids[4 * v + 1] = (int32_t)ix.y;
                ids[4 * v + 2] = (int32_t)ix.z; ids[4 * v + 3] = (int32_t)ix.w;
            }
        }
        over = cnt == 0xFFFFFFFFu;
        big = !over && cnt > (uint32_t)(GROUP * REG_CAND);
        const int rest = over ? 0 : (int)cnt - sub * REG_CAND;
        mine = rest < 0 ? 0 : (rest > REG_CAND ? REG_CAND : rest);
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) keys[i] = i < mine ? keys[i] + 1u : 0u;
    }
    // range of the candidates and the flags, in one workgroup round
    uint32_t kmax = 0u;
#pragma unroll
    for (int i = 0; i < REG_CAND; ++i) kmax = keys[i] > kmax ? keys[i] : kmax;
    kmax = wave_max_u32(kmax);
    t_lo = wave_max_u32(t_lo);
    const bool w_over = __ballot(over) != 0, w_big = __ballot(big) != 0;
    if (lane == 0) {
        ms.red[0][wave] = kmax;
        ms.red[1][wave] = t_lo;
        ms.red[2][wave] = (w_over ? 1u : 0u) | (w_big ? 2u : 0u);
    }
    __syncthreads();
    kmax = lds_max_u32<NT / 64>(ms.red[0]);
    t_lo = lds_max_u32<NT / 64>(ms.red[1]);
    uint32_t flags;
    {
        const uint32_t f = ms.red[2][lane < NT / 64 ? lane : 0];
        flags = (__ballot(f & 1u) != 0 ? 1u : 0u) | (__ballot(f & 2u) != 0 ? 2u : 0u);
    }
    if (flags & 1u) {
        return false;
    }
    if (flags & 2u) {
        // general mode: exclusive prefix of candidate counts, then equal runs
        int bad = 0;
        uint32_t carry = 0, tl = 1;
        for (int c0 = 0; c0 < p.n_chunks; c0 += NT) {
            const int c = c0 + tid;
            uint32_t n = 0;
            if (c < p.n_chunks) {
                n = meta[2 * c];
                const uint32_t th = meta[2 * c + 1] + 1u;
                tl = th > tl ? th : tl;
            }
            if (n == 0xFFFFFFFFu) {
                bad = 1;
                n = 0;
            }
            uint32_t tot;
            const uint32_t inc = block_scan<NT>(n, sm, &tot);
            if (c < p.n_chunks) pre[c] = carry + inc - n;
            carry += tot;
            __syncthreads();
        }
        if (tid == 0) pre[p.n_chunks] = carry;
        const uint32_t total = carry;
        const uint32_t per = (total + NT - 1) / NT;
        __syncthreads();
        if (__syncthreads_or(bad) || per > REG_CAND) {
            return false;
        }
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
        uint32_t km = 0u;
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            keys[i] = 0u;
            ids[i] = -1;
            const uint32_t f = lo + i;
            if (f < hi) {
                while (pre[c + 1] <= f) ++c;
                const size_t slot = ((size_t)q * p.n_chunks + c) * p.region_cap + (f - pre[c]);
                keys[i] = p.reg_key[slot] + 1u;
                ids[i] = p.reg_idx[slot];
                km = keys[i] > km ? keys[i] : km;
            }
        }
        mine = (int)(hi - lo);
        km = wave_max_u32(km);
        tl = wave_max_u32(tl);
        if (lane == 0) {
            ms.red[0][wave] = km;
            ms.red[1][wave] = tl;
        }
        __syncthreads();
        kmax = lds_max_u32<NT / 64>(ms.red[0]);
        t_lo = lds_max_u32<NT / 64>(ms.red[1]);
    }
    if (kmax < t_lo) return false;  // no candidate at or above T_lo
    // candidates below T_lo never decide anything: empty their slots
#pragma unroll
    for (int i = 0; i < REG_CAND; ++i) keys[i] = keys[i] >= t_lo ? keys[i] : 0u;

    // k-th key (kth) and how many keys equal to it are taken (need_ties)
    uint32_t need = (uint32_t)kk, kth = kmax, need_ties = need;
    uint32_t hi_bits = kmax;  // bits at and above `top` are settled
    const uint32_t diff = kmax ^ t_lo;
    int top = diff ? 32 - __builtin_clz(diff) : 0;
    int buf = 0;
    bool first = true;
    for (;;) {
        if (top == 0) {
            // every remaining key equals hi_bits; on the first pass count them
            if (first) {
                uint32_t n = 0;
#pragma unroll
                for (int i = 0; i < REG_CAND; ++i) n += keys[i] == kmax;
                uint32_t tot;
                scan_buf<NT>(n, ms, buf, &tot);
                if (tot < need) {
                    return false;
                }
                buf ^= 1;
            }
            kth = hi_bits;
            need_ties = need;
            break;
        }
        fence_keys(keys);
        const int s = top > MBITS ? top - MBITS : 0;
        const uint32_t mhi = top >= 32 ? 0u : (0xFFFFFFFFu << top);
        const uint32_t dmask = (1u << (top - s)) - 1u;
        if (!first) __syncthreads();  // the bins were zeroed by their owners
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            const bool in = (keys[i] & mhi) == (hi_bits & mhi) && keys[i] != 0u;
            atomicAdd(&ms.hist[in ? (keys[i] >> s) & dmask : MBINS + lane], 1u);
        }
        __syncthreads();
        uint32_t bin, above, in_bin, total;
        merge_find<NT>(ms, need, buf, &bin, &above, &in_bin, &total);
        buf ^= 1;
        if (first && total < need) {  // the k-th key lies below T_lo
            return false;
        }
        first = false;
        need -= above;
        hi_bits = (hi_bits & mhi) | (bin << s);
        top = s;
        if (top == 0) {
            kth = hi_bits;
            need_ties = need;
            break;
        }
        if (in_bin <= (uint32_t)RESOLVE_MAX) {
            // gather the bin into LDS: a wave takes its slots with one
            // addition to an LDS counter (the ranking does not depend on
            // the list's order) ...
            fence_keys(keys);
            const uint32_t m2 = 0xFFFFFFFFu << top;
            uint32_t n = 0;
#pragma unroll
            for (int i = 0; i < REG_CAND; ++i) n += (keys[i] & m2) == hi_bits && keys[i] != 0u;
            const uint32_t x = wave_inclusive_scan(n);
            const uint32_t w_n = (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
            uint32_t base = 0;
            if (w_n != 0u && lane == 0) base = atomicAdd(&ms.misc[3], w_n);
            uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)base, 0) + x - n;
            fence_keys(keys);
#pragma unroll
            for (int i = 0; i < REG_CAND; ++i) {
                const bool in = (keys[i] & m2) == hi_bits && keys[i] != 0u;
                ms.list[in ? slot : RESOLVE_MAX + lane] = keys[i];
                slot += in;
            }
            __syncthreads();
            // ... and rank it: PARTS threads share an element, part p comparing
            // it with list entries p, p + PARTS, ...; waves whose elements all
            // lie past the bin's end skip the ranking
            constexpr int PARTS = NT / RESOLVE_MAX;
            constexpr int EPW = 64 / PARTS;  // elements per wave
            if ((uint32_t)(wave * EPW) < in_bin) {
                const int e = tid / PARTS, part = tid % PARTS;
                const uint32_t mk = ms.list[e];
                const int n_j = (int)((in_bin + PARTS - 1) / PARTS);
                uint32_t gt = 0, ge = 0;
                for (int j = 0; j < n_j; ++j) {
                    const int o = j * PARTS + part;
                    const uint32_t ok = ms.list[o];
                    const bool in = (uint32_t)o < in_bin;
                    gt += in && ok > mk;
                    ge += in && ok >= mk;
                }
#pragma unroll
                for (int off = 1; off < PARTS; off <<= 1) {
                    gt += __shfl_xor(gt, off, 64);
                    ge += __shfl_xor(ge, off, 64);
                }
                // every element equal to the k-th key writes the same pair
                if (part == 0 && (uint32_t)e < in_bin && gt < need && need <= ge) {
                    ms.misc[0] = mk;
                    ms.misc[1] = need - gt;
                }
            }
            __syncthreads();
            kth = uniform_u32(ms.misc[0]);
            need_ties = uniform_u32(ms.misc[1]);
            break;
        }
    }

    fence_keys(keys);
    // keys > kth, and the first need_ties keys == kth in id order; one scan of
    // (greater << 16 | equal) gives both offsets (each total is below 2^16)
    uint32_t ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < REG_CAND; ++i) {
        ngt += keys[i] > kth;
        neq += keys[i] == kth;
    }
    const uint32_t packed = (ngt << 16) | neq;
    uint32_t tot;
    const uint32_t ex = scan_buf<NT>(packed, ms, buf, &tot) - packed;
    fence_keys(keys);
    uint32_t tb = ex & 0xFFFFu;
    uint32_t pos = (ex >> 16) + (tb < need_ties ? tb : need_ties);
    // up to STAGE_MAX selections are staged in LDS (ids in the free histogram)
    // and written out in order by consecutive lanes
    const bool stage = kk <= STAGE_MAX;
    uint32_t *st_id = ms.hist;
    if (stage) {
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            const bool eq = keys[i] == kth;
            const bool take = keys[i] > kth || (eq && tb < need_ties);
            tb += eq;
            const uint32_t a = take ? pos : STAGE_MAX + lane;
            st_id[a] = (uint32_t)ids[i];
            if (osc) ms.stage_key[a] = keys[i];  // scores are optional
            pos += take;
        }
    } else {
#pragma unroll
        for (int i = 0; i < REG_CAND; ++i) {
            bool take = keys[i] > kth;
            if (keys[i] == kth) take = (tb++ < need_ties);
            if (take) {
                oidx[pos] = ids[i];
                if (osc) osc[pos] = key_score(keys[i] - 1u);
                ++pos;
            }
        }
    }
    if (stage) {
        __syncthreads();
        for (int i = tid; i < kk; i += NT) {
            oidx[i] = (int32_t)st_id[i];
            if (osc) osc[i] = key_score(ms.stage_key[i] - 1u);
        }
    }
    return true;
}

template <int MODE, int NT>
__global__ __launch_bounds__(NT) void index_merge_kernel(IndexPlan p) {
    extern __shared__ uint32_t dyn[];
    __shared__ IdxSmem sm;
    __shared__ MergeSmem<NT> ms;
    const int q = blockIdx.x, tid = threadIdx.x;
    const int b = q / p.Tq;
    uint32_t *pre = dyn;                                  // [n_chunks + 1] candidate offsets
    uint32_t *skey = dyn + p.n_chunks + 1;                // [chunk] (exact fallback)
    float *sq = (float *)(skey + p.chunk);                // f32 mode query
#pragma unroll
    for (int v = 0; v < MBINS / NT / 4; ++v) *(uint4 *)&ms.hist[MBINS / NT * tid + 4 * v] = make_uint4(0, 0, 0, 0);
    if (MODE == 0) {
        const float *iq = (const float *)p.iq + (size_t)q * p.H * p.dI;
        for (int i = tid; i < p.H * p.dI; i += NT) sq[i] = iq[i];
    }
    const int64_t nvis = visible_entries(p, q);
    const int kk = (int)(nvis < p.k ? nvis : p.k);
    int32_t *oidx = p.out_idx + (size_t)q * p.k;
    float *osc = p.out_score ? p.out_score + (size_t)q * p.k : nullptr;
    for (int i = kk + tid; i < p.k; i += NT) {
        oidx[i] = -1;
        if (osc) osc[i] = 0.f;
    }
    if (kk == 0) return;
    if (!merge_select<NT>(p, q, kk, pre, sm, ms)) exact_fallback<MODE, NT>(p, q, b, nvis, kk, skey, sq, sm);
}

template <int MODE>
static void launch_mode(const IndexPlan &p, hipStream_t s) {
    const size_t q_lds = MODE == 0 ? (size_t)p.H * p.dI * 4 : 0;
    // several queries per sequence over many entries (chunked prefill): the
    // layout's chunks are IDX_CPW sub-chunks, one workgroup each
    const bool cpw = p.chunk > IDX_CHUNK;
    for (int q0 = 0; q0 < p.Q; q0 += MAX_GRID_Y) {
        IndexPlan ps = p;
        ps.q_base = q0;
        const int nq = p.Q - q0 < MAX_GRID_Y ? p.Q - q0 : MAX_GRID_Y;
        if (cpw)
            hipLaunchKernelGGL(index_score_cpw_kernel<MODE == 0 ? 1 : MODE>, dim3(p.n_chunks, nq), dim3(IT),
                               (size_t)p.chunk * 4 + (size_t)p.H * 72, s, ps);
        else
            hipLaunchKernelGGL(index_score_kernel<MODE>, dim3(p.n_chunks, nq), dim3(IT), (size_t)p.chunk * 4 + q_lds, s,
                               ps);
    }
    // Few queries (decode): 1,024 threads per query, whose sixteen waves hide
    // a lone workgroup's latencies; many (chunked prefill): 512, so that two
    // workgroups share a compute unit.
    const size_t m_lds = (size_t)(p.n_chunks + 1 + p.chunk) * 4 + q_lds;
    if (p.Q >= MERGE_WIDE_Q) hipLaunchKernelGGL((index_merge_kernel<MODE, 512>), dim3(p.Q), dim3(512), m_lds, s, p);
    else hipLaunchKernelGGL((index_merge_kernel<MODE, 1024>), dim3(p.Q), dim3(1024), m_lds, s, p);
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
