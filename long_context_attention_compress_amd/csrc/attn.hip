// sparse_window_attn / hca_attn: attention of H_q query heads (one shared KV
// head) over compressed entries plus the raw sliding window.
//
// [chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich nutzbar",
// section "Hybrid Attention: CSA und HCA"]: CSA attends over the top-k
// compressed blocks per query, HCA densely over all compressed blocks.
// [golem.de, "... Bei Deepseek V4 haben kleine Änderungen große Wirkung",
// section "Komprimierte Erinnerung für längere Kontexte"]: both add the
// uncompressed last 128 tokens; the first two layers use the window alone.
//
// Key list of query (b, i) at position t: [entries] ++ [window rows], one
// joint softmax. Entries are idx[q][0..k) (sparse) or 0..n_ent-1 (dense).
// Work is split along the key list: workgroup (split, query) handles keys
// [split*KS, split*KS + KS) and leaves (running max, running sum, unnormalised
// output) per head; a combine kernel merges the splits in a fixed order
// (deterministic). With one split the workgroup writes the output directly.
//
// FP8+BF16 path (D = 192: 128 E4M3 dims with one float32 scale + 64 BF16 RoPE
// dims), on MFMA V_MFMA_F32_16X16X32_BF16:
//  * S^T = K Q^T with keys as M and 16 heads per wave as N, so each lane ends
//    up owning one head; E4M3 codes convert exactly to BF16 and the row scale
//    multiplies the no-RoPE partial sum; the rotated RoPE query is split into
//    two BF16 terms (hi + lo) so it keeps ~16 mantissa bits.
//  * O^T += V^T P^T with dims as M: the lane's eight probabilities are already
//    the B operand (the key order inside the 32-wide contraction is permuted
//    to match); V is staged row-major in LDS and read transposed with
//    ds_read_b64_tr_b16; the V row scale is folded into P for the E4M3 dims,
//    and P goes in as two BF16 terms (hi + lo).
//  * All 64 heads of a workgroup share each staged K/V tile.
//  * The split's store rows are resolved into LDS first (one coalesced pass
//    over the selected ids); tile loads are branch-free and run two tiles
//    ahead of the tile being computed.
//  * The running max is raised lazily (only when a tile beats it by 2^8), so
//    the 48 accumulator registers are rarely rescaled.
//  * Fused window append (decode): the workgroup whose split holds the query
//    token's own key (the last window row) encodes the token's raw K and V
//    rows exactly as the m = 1 compressor does, writes them into the window
//    stores and stages them from LDS in place of the store's old contents;
//    this saves the separate append launch.

#include "common.hpp"

namespace v4a {

constexpr int AT = 256;
constexpr int TK = 32;  // keys per tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

// The key list of one query at position t. Counts and rows fit 32 bits: a
// list holds at most MAX_KEY_LIST keys and the stores fewer than 2^30 rows
// (the host checks both), so the per-key arithmetic below is 32-bit.
struct KeyInfo {
    int32_t n_list;  // entries in the list
    int32_t n_win;   // window rows
    int64_t t;
    int32_t wrow0;   // window-store row of the window's first key (position t - n_win + 1);
                     // a linear store's row count when that position lies past it
};

// Division of a position by a divisor fixed for the call (m, the ring):
// below 2^31 a multiply and a shift with host-made constants, the 64-bit
// division otherwise. The quotient is exact: with s' = 31 + ceil(log2 d) and
// M = ceil(2^s' / d), x M / 2^s' exceeds x / d by x (M d - 2^s') / (d 2^s'),
// which is below 1 / d (x < 2^31 and M d - 2^s' < d <= 2^(s' - 31)), too
// little to reach the next integer.
__device__ __forceinline__ int64_t div_fixed(int64_t x, int64_t d, uint32_t mul, uint32_t sh) {
    return (uint64_t)x < (1ull << 31) ? (int64_t)(((uint64_t)x * mul) >> sh) : x / d;
}

// Host side: the multiplier and shift of div_fixed for 1 <= d < 2^31.
inline void div_consts(int64_t d, uint32_t *mul, uint32_t *sh) {
    int s = 0;
    while (((int64_t)1 << s) < d) ++s;
    const int k = 31 + s;
    const unsigned __int128 num = (unsigned __int128)1 << k;
    *mul = (uint32_t)((num + (unsigned __int128)d - 1) / (unsigned __int128)d);
    *sh = (uint32_t)k;
}

__device__ __forceinline__ KeyInfo key_info(const KeyConsts &kc, int64_t t) {
    KeyInfo ki;
    ki.t = t;
    ki.wrow0 = 0;
    if (ki.t < 0) {
        ki.n_list = 0;
        ki.n_win = 0;
        return ki;
    }
    ki.n_win = (int32_t)(ki.t + 1 < kc.W ? ki.t + 1 : kc.W);
    const int64_t pos0 = ki.t - ki.n_win + 1;
    int64_t wrow0 = pos0;
    if (kc.ring > 0) wrow0 = pos0 - div_fixed(pos0, kc.ring, kc.r_mul, (kc.misc >> 16) & 0xff) * kc.ring;
    ki.wrow0 = (int32_t)(wrow0 < kc.wrows ? wrow0 : kc.wrows);
    if (kc.misc & 1u) ki.n_list = kc.cap;
    else {
        const int64_t n = div_fixed(ki.t + 1, kc.m, kc.m_mul, (kc.misc >> 8) & 0xff);
        ki.n_list = (int32_t)(n < kc.cap ? n : kc.cap);
    }
    return ki;
}

// Store row of key j of the list; -1 when the slot holds no key. *win: from the window stores.
__device__ __forceinline__ int64_t key_row(const AttnPlan &p, int q, const KeyInfo &ki, int64_t j, bool *win) {
    if (j < ki.n_list) {
        *win = false;
        int64_t e = p.sparse ? (int64_t)p.idx[(size_t)q * p.k + j] : j;
        return (e >= 0 && e < p.ek.rows) ? e : -1;
    }
    *win = true;
    int64_t w = j - ki.n_list;
    if (w >= ki.n_win) return -1;
    int64_t pos = ki.t - ki.n_win + 1 + w;
    int64_t row = p.wk.ring > 0 ? pos % p.wk.ring : pos;
    return row < p.wk.rows ? row : -1;
}

constexpr int32_t WIN_BIT = 1 << 30;  // a row code with this bit set is a window-store row

// Row code of key j of the list: the store row, WIN_BIT set for a window row,
// -1 for a slot without a key. `id` is the selected id when j is a sparse
// list entry (unused otherwise). The same function serves the per-split rows
// table and the rows of the first two tiles, which are resolved per lane.
// Both candidates are formed and one is selected (no per-lane branches).
__device__ __forceinline__ int32_t key_code(const KeyConsts &kc, const KeyInfo &ki, int32_t j, int32_t id) {
    const int32_t e = (kc.misc & 1u) ? id : j;
    const int32_t ec = (uint32_t)e < (uint32_t)kc.erows ? e : -1;
    // window key w at position t - n_win + 1 + w; its ring row without a
    // division: w < n_win <= ring, so one wrap at most
    const int32_t w = j - ki.n_list;
    int32_t row = ki.wrow0 + w;
    row = (kc.ring > 0 && row >= kc.ring) ? row - kc.ring : row;
    const int32_t wc = ((uint32_t)w < (uint32_t)ki.n_win && row < kc.wrows) ? (row | WIN_BIT) : -1;
    return j < ki.n_list ? ec : wc;
}

// ------------------------------------------------------------------ F32 ----
// fp32 VALU path (the small fp32 configuration). H*D <= 4096.

constexpr int F32_OUT = 16;  // outputs (h, d) per thread

__global__ __launch_bounds__(AT) void attn_f32_kernel(AttnPlan p) {
    extern __shared__ float fsm[];
    const int H = p.H, D = p.D;
    float *sq = fsm;                  // [H][D] rotated query
    float *sk = sq + H * D;           // [TK][D]
    float *sv = sk + TK * D;          // [TK][D]
    float *ss = sv + TK * D;          // [H][TK]
    float *corr = ss + H * TK;        // [H]
    float *mrun = corr + H;           // [H]
    float *lrun = mrun + H;           // [H]
    const int tid = threadIdx.x;
    const int q = blockIdx.y + p.q_base, split = blockIdx.x;
    const int b = q / p.Tq;
    const KeyInfo ki = key_info(p.kc, p.q_pos[q]);
    const float *qin = (const float *)p.q + (size_t)q * H * D;
    const int Dn = D - ROPE_DIM;
    for (int i = tid; i < H * D; i += AT) {
        const int h = i / D, d = i % D;
        float v = qin[i];
        if (d >= Dn) {
            const int r = d - Dn, pr = r >> 1;
            double sn, cs;
            rope_sincos((double)ki.t * p.inv_freq[pr], &sn, &cs);
            const double x = qin[h * D + Dn + 2 * pr], y = qin[h * D + Dn + 2 * pr + 1];
            v = (float)((r & 1) ? x * sn + y * cs : x * cs - y * sn);
        }
        sq[i] = v;
    }
    for (int h = tid; h < H; h += AT) {
        mrun[h] = -__builtin_inff();
        lrun[h] = 0.f;
    }
    float acc[F32_OUT];
#pragma unroll
    for (int i = 0; i < F32_OUT; ++i) acc[i] = 0.f;
    const float sc2 = p.sm_scale * 1.4426950408889634f;
    const int64_t n_keys = ki.n_list + ki.n_win;
    const int64_t j0 = (int64_t)split * p.keys_per_split;
    const int64_t j1 = j0 + p.keys_per_split < n_keys ? j0 + p.keys_per_split : n_keys;
    __syncthreads();
    for (int64_t jt = j0; jt < j1; jt += TK) {
        for (int i = tid; i < TK * D; i += AT) {
            const int r = i / D, d = i % D;
            bool win;
            const int64_t row = (jt + r < j1) ? key_row(p, q, ki, jt + r, &win) : -1;
            float kv = 0.f, vv = 0.f;
            if (row >= 0) {
                const KvView &K = win ? p.wk : p.ek;
                const KvView &V = win ? p.wv : p.ev;
                kv = ((const float *)(K.f32 + b * K.f32_bs + row * K.f32_rs))[d];
                vv = ((const float *)(V.f32 + b * V.f32_bs + row * V.f32_rs))[d];
            }
            sk[i] = kv;
            sv[i] = vv;
        }
        __syncthreads();
        for (int i = tid; i < H * TK; i += AT) {
            const int h = i / TK, r = i % TK;
            bool win;
            const int64_t row = (jt + r < j1) ? key_row(p, q, ki, jt + r, &win) : -1;
            float s = -__builtin_inff();
            if (row >= 0) {
                float dot = 0.f;
                for (int d = 0; d < D; ++d) dot = __builtin_fmaf(sq[h * D + d], sk[r * D + d], dot);
                s = dot * sc2;
            }
            ss[i] = s;
        }
        __syncthreads();
        for (int h = tid; h < H; h += AT) {
            float mx = -__builtin_inff();
            for (int r = 0; r < TK; ++r) mx = __builtin_fmaxf(mx, ss[h * TK + r]);
            const float mo = mrun[h];
            const float mn = __builtin_fmaxf(mo, mx);
            float c = 1.f, sum = 0.f;
            if (mn != -__builtin_inff()) {
                c = exp2f(mo - mn);
                for (int r = 0; r < TK; ++r) {
                    const float e = exp2f(ss[h * TK + r] - mn);
                    ss[h * TK + r] = e;
                    sum += e;
                }
            } else {
                for (int r = 0; r < TK; ++r) ss[h * TK + r] = 0.f;
            }
            corr[h] = c;
            mrun[h] = mn;
            lrun[h] = lrun[h] * c + sum;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < F32_OUT; ++i) {
            const int o = tid + AT * i;
            if (o < H * D) {
                const int h = o / D, d = o % D;
                float a = acc[i] * corr[h];
                for (int r = 0; r < TK; ++r) a = __builtin_fmaf(ss[h * TK + r], sv[r * D + d], a);
                acc[i] = a;
            }
        }
        __syncthreads();
    }
    // epilogue
#pragma unroll
    for (int i = 0; i < F32_OUT; ++i) {
        const int o = tid + AT * i;
        if (o >= H * D) continue;
        const int h = o / D, d = o % D;
        if (p.n_split == 1) {
            const float l = lrun[h];
            ((float *)p.o)[(size_t)q * H * D + o] = l > 0.f ? acc[i] / l : 0.f;
            if (d == 0 && p.lse)
                p.lse[(size_t)q * H + h] = l > 0.f ? (mrun[h] + log2f(l)) * 0.6931471805599453f : -__builtin_inff();
        } else {
            const size_t base = ((size_t)q * p.n_split + split) * H;
            p.part_o[(base + h) * D + d] = acc[i];
            if (d == 0) {
                p.part_ml[(base + h) * 2] = mrun[h];
                p.part_ml[(base + h) * 2 + 1] = lrun[h];
            }
        }
    }
}

// ----------------------------------------------------------- FP8 + BF16 ----

constexpr int MD = 192;         // head dim
constexpr int MDN = 128;        // E4M3 dims
constexpr int KB_LD = MD + 8;   // bf16 elements per staged K or V row (padded)
constexpr int MAX_KS = 2048;    // keys per split (their store rows are resolved into LDS first)

// One staged tile: K and V row-major BF16 (V read transposed by
// ds_read_b64_tr_b16), per-key scales and the empty-slot bias.
struct TileBuf {
    __bf16 kb[TK * KB_LD];
    __bf16 vb[TK * KB_LD];
    float ksc[TK] __attribute__((aligned(16)));    // K row scale of each key (0 for an empty slot)
    float kbias[TK] __attribute__((aligned(16)));  // 0, or -inf for an empty slot
    float vsc[TK] __attribute__((aligned(16)));
};

// The row of a fused window append, encoded as the stores hold it: E4M3
// codes and BF16 RoPE pairs of K and V, and the two row scales.
struct AppRow {
    uint8_t kc[MDN] __attribute__((aligned(16)));
    uint8_t kr[2 * ROPE_DIM] __attribute__((aligned(16)));
    uint8_t vc[MDN] __attribute__((aligned(16)));
    uint8_t vr[2 * ROPE_DIM] __attribute__((aligned(16)));
    float ksc, vsc;
};

// NS key streams per workgroup, each with two tile buffers (one is computed
// while the next tile is staged into the other); at the end the streams'
// partial results meet in the (then free) tile buffers.
template <int NS>
struct MxSmem {
    TileBuf tb[NS][2];
    double rcos[ROPE_PAIRS];   // RoPE at the query position, float64 (the fused append's key rotation)
    double rsin[ROPE_PAIRS];
    float2 rsc[ROPE_PAIRS];    // the same (sin, cos) rounded to float32 (the query rotation)
    int32_t rows[MAX_KS];       // row of each key of the split; bit 30 marks a window row; -1: no key
    float xml[NS > 1 ? 2 * AT : 1];
    AppRow app;
    uint32_t sync[NS];         // per-stream round counters (two streams)
};

// A tile in flight: the raw loads and which of them hold a key. Slots without
// a key are zeroed only when the tile is staged, so that issuing the next
// tile's loads never waits for this one's data.
// Thread t of a stream loads row t / 8 of the tile: the 16-byte piece t % 8
// of its E4M3 codes (16 codes) and of its BF16 RoPE dims (8 values), for K
// and for V, so every lane converts codes when the tile is staged.
struct TileRegs {
    v4i kn, kr, vn, vr;
    float sc;
    bool ok, sok;
};

// One batch element's planes of one store, with their row strides. Built
// once per workgroup from the (uniform) plan, so that choosing between the
// entry and the window store per lane is a register select and never a load
// of the plan's fields through a per-lane address.
struct Planes {
    const char *nope, *rope, *scale;
    int64_t nope_rs, rope_rs, scale_rs;
};
__device__ __forceinline__ Planes planes_of(const KvView &s, int b) {
    Planes r;
    r.nope = s.nope + b * s.nope_bs;
    r.rope = s.rope + b * s.rope_bs;
    r.scale = s.scale + b * s.scale_bs;
    r.nope_rs = s.nope_rs;
    r.rope_rs = s.rope_rs;
    r.scale_rs = s.scale_rs;
    return r;
}
struct TileSrc {
    Planes ek, ev, wk, wv;
};

template <typename T>
__device__ __forceinline__ T pick(bool c, T a, T b) { return c ? a : b; }

// What a lane loads of every tile, fixed for the whole kernel: the row-0
// addresses of its pieces in each store's planes (no-RoPE codes, RoPE pairs)
// and the planes' row strides, and (lanes of threads 0..63) the scale plane
// of K (threads < 32) or V. Per tile only the row changes, so a load costs
// one select of the store and one 32 x 32 + 64-bit multiply-add.
struct LaneSrc {
    const char *kwn, *ken, *kwr, *ker, *vwn, *ven, *vwr, *ver;
    uint32_t kwn_s, ken_s, kwr_s, ker_s, vwn_s, ven_s, vwr_s, ver_s;
    const char *sw, *se;
    uint32_t srw, sre;
};
__device__ __forceinline__ LaneSrc lane_src(const TileSrc &S, int tid) {
    const int off = 16 * (tid & 7);
    LaneSrc L;
    L.kwn = S.wk.nope + off; L.ken = S.ek.nope + off; L.kwr = S.wk.rope + off; L.ker = S.ek.rope + off;
    L.vwn = S.wv.nope + off; L.ven = S.ev.nope + off; L.vwr = S.wv.rope + off; L.ver = S.ev.rope + off;
    L.kwn_s = (uint32_t)S.wk.nope_rs; L.ken_s = (uint32_t)S.ek.nope_rs;
    L.kwr_s = (uint32_t)S.wk.rope_rs; L.ker_s = (uint32_t)S.ek.rope_rs;
    L.vwn_s = (uint32_t)S.wv.nope_rs; L.ven_s = (uint32_t)S.ev.nope_rs;
    L.vwr_s = (uint32_t)S.wv.rope_rs; L.ver_s = (uint32_t)S.ev.rope_rs;
    const bool isk = tid < TK;
    L.sw = pick(isk, S.wk.scale, S.wv.scale);
    L.se = pick(isk, S.ek.scale, S.ev.scale);
    L.srw = (uint32_t)pick(isk, S.wk.scale_rs, S.wv.scale_rs);
    L.sre = (uint32_t)pick(isk, S.ek.scale_rs, S.ev.scale_rs);
    return L;
}

__device__ __forceinline__ const char *row_addr(const char *base, uint32_t row, uint32_t stride) {
    return base + (uint64_t)row * stride;
}

// Issue the loads of one 32-key tile. Branch-free: a slot without a key
// (also every slot of a tile past the split's end) reads row 0 of the window
// store (always present; the same line for the whole wave, so a cache hit)
// and is zeroed when staged. Every call issues the same five loads, so the
// wait before staging a tile counts exactly the loads issued after it and
// leaves the next tile's loads in flight; with a branch around the loads the
// compiler can only wait for all of them.
// `code`: row code of the lane's row, `cs`: of the key whose scale the lane
// loads (threads 0..31: K scale of key tid, 32..63: V scale of key tid - 32;
// -1 for the other threads).
// NT: non-temporal loads (one query token per sequence: no other workgroup
// reads the rows again soon); ordinary loads otherwise (several tokens per
// sequence: neighbouring tokens' workgroups read mostly the same rows). Each
// form measured faster for its case (43-layer decode stack 1.23 against
// 1.28 ms; chunked prefill 8.50 against 8.60 ms per pass).
template <bool NT>
__device__ __forceinline__ v4i ld_row(const char *a) {
    return NT ? __builtin_nontemporal_load((const v4i *)a) : *(const v4i *)a;
}

template <bool NT>
__device__ __forceinline__ void load_tile_codes(const LaneSrc &L, int32_t code, int32_t cs, TileRegs &R) {
    const bool ok = code >= 0;
    const bool win = !ok || (code & WIN_BIT);
    const uint32_t row = ok ? (uint32_t)(code & (WIN_BIT - 1)) : 0u;
    R.kn = ld_row<NT>(row_addr(pick(win, L.kwn, L.ken), row, pick(win, L.kwn_s, L.ken_s)));
    R.kr = ld_row<NT>(row_addr(pick(win, L.kwr, L.ker), row, pick(win, L.kwr_s, L.ker_s)));
    R.vn = ld_row<NT>(row_addr(pick(win, L.vwn, L.ven), row, pick(win, L.vwn_s, L.ven_s)));
    R.vr = ld_row<NT>(row_addr(pick(win, L.vwr, L.ver), row, pick(win, L.vwr_s, L.ver_s)));
    R.ok = ok;
    const bool oks = cs >= 0;
    const bool wins = !oks || (cs & WIN_BIT);
    const uint32_t rows_ = oks ? (uint32_t)(cs & (WIN_BIT - 1)) : 0u;
    R.sc = *(const float *)row_addr(pick(wins, L.sw, L.se), rows_, pick(wins, L.srw, L.sre));
    R.sok = oks;
}

// The same from the split's rows table (LDS).
template <bool NT>
__device__ __forceinline__ void load_tile(const LaneSrc &L, const int32_t *rows, int rel, int n_rel, TileRegs &R,
                                          int tid) {
    const int r = tid >> 3, rs = tid & (TK - 1);
    const int32_t code = rel + r < n_rel ? rows[rel + r] : -1;
    const int32_t cs = (tid < 2 * TK && rel + rs < n_rel) ? rows[rel + rs] : -1;
    load_tile_codes<NT>(L, code, cs, R);
}

template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
    bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(unsigned, v);
}

// 16 E4M3 codes -> 16 BF16 values (exact), written as two 16-byte LDS stores
__device__ __forceinline__ void store_codes(__bf16 *dst, const v4i &c) {
    v4i lo, hi;
    lo[0] = fp8x2_to_bf16x2<false>(c[0]);
    lo[1] = fp8x2_to_bf16x2<true>(c[0]);
    lo[2] = fp8x2_to_bf16x2<false>(c[1]);
    lo[3] = fp8x2_to_bf16x2<true>(c[1]);
    hi[0] = fp8x2_to_bf16x2<false>(c[2]);
    hi[1] = fp8x2_to_bf16x2<true>(c[2]);
    hi[2] = fp8x2_to_bf16x2<false>(c[3]);
    hi[3] = fp8x2_to_bf16x2<true>(c[3]);
    *(v4i *)dst = lo;
    *(v4i *)(dst + 8) = hi;
}

// `cur`: the split-relative key of a fused append (-1: none). The threads
// that stage its slot then overwrite it with the encoded row from LDS (the
// same threads, so the later store wins), in place of the loaded (previous)
// store contents.
// `ksc_mul` multiplies the K row scales as they are staged (the softmax scale
// in log2 units, so that a score is one fma).
__device__ __forceinline__ void stage_tile(const TileRegs &R, const int32_t *rows, TileBuf &sm, int rel, int n_rel,
                                           int tid, const AppRow &app, int cur, float ksc_mul) {
    const int r = tid >> 3, part = tid & 7;
    const v4i z = {0, 0, 0, 0};
    const v4i kn = R.ok ? R.kn : z, vn = R.ok ? R.vn : z, kr = R.ok ? R.kr : z, vr = R.ok ? R.vr : z;
    store_codes(&sm.kb[r * KB_LD + 16 * part], kn);
    store_codes(&sm.vb[r * KB_LD + 16 * part], vn);
    *(v4i *)&sm.kb[r * KB_LD + MDN + 8 * part] = kr;
    *(v4i *)&sm.vb[r * KB_LD + MDN + 8 * part] = vr;
    // The empty asm makes the loaded scale opaque here, at staging time:
    // without it the compiler folds this select into the branch that issued
    // the load and waits for the load there, before the next tile's loads
    // are issued.
    float sc = R.sc;
    asm volatile("" : "+v"(sc));
    sc = R.sok ? sc : 0.f;
    if (tid < TK) {
        sm.ksc[tid] = sc * ksc_mul;
        sm.kbias[tid] = (rel + tid < n_rel && rows[rel + tid] >= 0) ? 0.f : -__builtin_inff();
    } else if (tid < 2 * TK) {
        sm.vsc[tid - TK] = sc;
    }
    if (cur >= rel && cur < rel + TK) {  // uniform: this tile holds the appended key
        const int ra = cur - rel;
        if (r == ra) {
            store_codes(&sm.kb[ra * KB_LD + 16 * part], *(const v4i *)&app.kc[16 * part]);
            store_codes(&sm.vb[ra * KB_LD + 16 * part], *(const v4i *)&app.vc[16 * part]);
            *(v4i *)&sm.kb[ra * KB_LD + MDN + 8 * part] = *(const v4i *)&app.kr[16 * part];
            *(v4i *)&sm.vb[ra * KB_LD + MDN + 8 * part] = *(const v4i *)&app.vr[16 * part];
        }
        if (tid == ra) sm.ksc[ra] = app.ksc * ksc_mul;
        if (tid == TK + ra) sm.vsc[ra] = app.vsc;
    }
}

__device__ __forceinline__ bf16x8 ld16(const __bf16 *p) { return *(const bf16x8 *)p; }

// Two floats as hi + lo BF16 terms (hi = RNE(x), lo = RNE(x - hi)) into
// elements e, e+1 of hi and lo, one conversion instruction per pair.
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The combines read the split partials once, with non-temporal loads: with
// ordinary loads the 7-10 MB of a decode call's partials stayed in the L2s,
// and the decode step took 2.6 us longer (the combine itself and the next
// kernels, measured).
__device__ __forceinline__ float2 ld_ml(const float *a) {
    const f32x2 v = __builtin_nontemporal_load((const f32x2 *)a);
    return make_float2(v[0], v[1]);
}
__device__ __forceinline__ void split_bf16x2(float a, float b, bf16x8 &hi, bf16x8 &lo, int e) {
    const bf16x2 h = __builtin_convertvector((f32x2){a, b}, bf16x2);
    const bf16x2 l = __builtin_convertvector((f32x2){a - (float)h[0], b - (float)h[1]}, bf16x2);
    hi[e] = h[0];
    hi[e + 1] = h[1];
    lo[e] = l[0];
    lo[e + 1] = l[1];
}

// V^T operand of the P.V product: lane (group g, position j) gets, for dim
// 16*dt + j, the keys of its contraction slots: 4g..4g+3 and 16+4g..16+4g+3.
// Each ds_read_b64_tr_b16 transposes a 16x4 block within the 16-lane group:
// source lane 4k+r reads key kappa(k), dims 16*dt + 4r .. +3.
typedef short v4s __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 vt_operand(const TileBuf &sm, int dt, int g, int j) {
    const int k = j >> 2, r = j & 3;
    const __bf16 *a = &sm.vb[(4 * g + k) * KB_LD + 16 * dt + 4 * r];
    const __bf16 *c = &sm.vb[(16 + 4 * g + k) * KB_LD + 16 * dt + 4 * r];
    v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)a);
    v4s y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)c);
    v4i r4 = {(int)((unsigned short)x[0] | ((unsigned)(unsigned short)x[1] << 16)),
              (int)((unsigned short)x[2] | ((unsigned)(unsigned short)x[3] << 16)),
              (int)((unsigned short)y[0] | ((unsigned)(unsigned short)y[1] << 16)),
              (int)((unsigned short)y[2] | ((unsigned)(unsigned short)y[3] << 16))};
    return __builtin_bit_cast(bf16x8, r4);
}

__device__ __forceinline__ float swap16_max(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
}

// The running maximum is raised only when a tile's maximum exceeds it by more
// than 2^RESCALE_SLACK (then the accumulators are rescaled); in between, the
// probabilities may exceed 1 by at most that factor, which float32 absorbs.
constexpr float RESCALE_SLACK = 8.0f;

// NS key streams: the workgroup has NS x 256 threads; stream s takes tiles
// s, s + NS, ... of the split with its own four waves (16 heads each) and
// tile buffer, so NS tiles are in flight per head group. The streams' online
// softmax states are merged at the end. NT: non-temporal K/V loads (one
// query token per sequence).
template <int NW, int NS, bool NT>
__global__ __launch_bounds__(AT * NS, 2) void attn_mx_kernel(AttnPlan p) {
    __shared__ MxSmem<NS> sm;
    const int tid = threadIdx.x, lane = tid & 63;
    const int stream = tid / AT, tids = tid % AT, wave = tids >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int q = blockIdx.y + p.q_base, split = blockIdx.x;
    const int b = q / p.Tq;
    const int H = p.H;
    const bool active = wave < NW;
    const int head = 16 * wave + col;
    // The key-list constants are read with the plan's lines and pinned in
    // scalar registers (the empty asm keeps the compiler from loading them
    // again where they are used, one wait per load, after the position).
    KeyConsts kc = p.kc;
    touch_args(p);  // every line of the plan in one scalar round trip
    asm volatile("" : "+s"(kc.W), "+s"(kc.ring), "+s"(kc.wrows), "+s"(kc.erows), "+s"(kc.cap), "+s"(kc.misc),
                 "+s"(kc.m_mul), "+s"(kc.r_mul), "+s"(kc.m));
    // The position (a pointer, then the value: the longest chain of the
    // prologue) is asked for first, as a vector load whose address the
    // compiler cannot prove uniform, and read into a scalar only where it is
    // first needed: that wait then leaves every load issued after it in
    // flight. (A load known to be uniform is read into a scalar at once, with
    // a wait for it right there; a scalar load's wait is shared with every
    // later scalar-cache and LDS wait.)
    int opaque_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque_zero));
    const int64_t t_lane = p.q_pos[q + opaque_zero];
    __builtin_amdgcn_sched_barrier(0);
    constexpr int IDS = MAX_KS / (AT * NS);
    const int64_t j0 = (int64_t)split * p.keys_per_split;
    // Id loads without per-lane branches (which would wait for each load in
    // turn): clamped positions, a dense call reading a valid dummy address; the
    // values are masked where they are used.
    const int32_t *ip = p.id_src + q * p.id_stride;
    const int64_t jmax = p.id_jmax;
    // The stream's first two tiles are loaded before the rows table exists:
    // each lane resolves the keys it needs itself (its row of each tile and,
    // threads 0..63, the key whose scale it loads) from ids asked for first,
    // so the tile loads leave as soon as the position is known.
    const int ra = TK * stream + (tids >> 3), rb = ra + TK * NS;
    const int sa = TK * stream + (tids & (TK - 1)), sb = sa + TK * NS;
    int32_t fid[4];
    {
        const int rr[4] = {ra, rb, sa, sb};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t j = j0 + rr[u];
            fid[u] = ip[j < jmax ? j : jmax];
        }
    }
    // the stores' planes and this lane's load sources (plan fields only)
    TileSrc src;
    src.wk = planes_of(p.wk, b);
    src.wv = planes_of(p.wv, b);
    src.ek = p.has_ent ? planes_of(p.ek, b) : src.wk;
    src.ev = p.has_ent ? planes_of(p.ev, b) : src.wv;
    const LaneSrc lsrc = lane_src(src, tids);
    // RoPE frequency of pair `lane & 31` (the table below is built by lanes
    // 0..31 of the first wave)
    const double ifreq = p.inv_freq[lane & 31];
    // The query and (sparse) this split's selected ids do not depend on the
    // query position: their loads are issued before the position arrives.
    const __bf16 *qp = (const __bf16 *)p.q + ((size_t)q * H + (active ? head : 0)) * MD;
    bf16x8 qn[4], qraw[2];
#pragma unroll
    for (int c = 0; c < 4; ++c) qn[c] = ld16(qp + 32 * c + 8 * g);
#pragma unroll
    for (int c = 0; c < 2; ++c) qraw[c] = ld16(qp + MDN + 32 * c + 8 * g);
    int32_t ids[IDS];
#pragma unroll
    for (int u = 0; u < IDS; ++u) {
        const int64_t j = j0 + tid + AT * NS * u;
        ids[u] = ip[j < jmax ? j : jmax];
    }
    const int64_t t_pos = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(t_lane >> 32)) << 32) |
                                    (uint32_t)__builtin_amdgcn_readfirstlane((int)t_lane));
    const KeyInfo ki = key_info(kc, t_pos);
    const int64_t n_keys = ki.n_list + ki.n_win;
    const int64_t j1 = j0 + p.keys_per_split < n_keys ? j0 + p.keys_per_split : n_keys;
    const int n_rel = j1 > j0 ? (int)(j1 - j0) : 0;
    TileRegs RA, RB;
    {
        auto first = [&](int rel, int32_t id) { return rel < n_rel ? key_code(kc, ki, (int32_t)j0 + rel, id) : -1; };
        const bool sl = tids < 2 * TK;  // threads 0..63 load the scales
        load_tile_codes<NT>(lsrc, first(ra, fid[0]), sl ? first(sa, fid[2]) : -1, RA);
        load_tile_codes<NT>(lsrc, first(rb, fid[1]), sl ? first(sb, fid[3]) : -1, RB);
    }
    // Fused window append: the token's own key is the last of the list (the
    // window row at t). The workgroup whose split holds it reads the token's
    // raw K and V rows, one 32-bit word (two BF16 values) per lane of its last
    // three waves: the last wave K's no-RoPE dims 2l, 2l + 1, the one before
    // V's, and the third last the RoPE pairs (K's on lanes 0..31, V's on
    // 32..63). Only these waves read them, so the rows are not a hot spot.
    const int aw = (AT * NS - 1 - tid) >> 6;
    const bool app_here = p.has_app && ki.n_win > 0 && n_keys - 1 >= j0 && n_keys - 1 < j1;  // uniform
    uint32_t araw = 0;
    if (app_here && aw < 3) {
        const uint32_t *rk = (const uint32_t *)(p.app_k + (size_t)q * MD);
        const uint32_t *rv = (const uint32_t *)(p.app_v + (size_t)q * MD);
        araw = aw == 0 ? rk[lane] : aw == 1 ? rv[lane] : lane < 32 ? rk[MDN / 2 + lane] : rv[MDN / 2 - 32 + lane];
    }
    // resolve the split's keys to store rows once (later tiles, the staging
    // masks), and the RoPE table
#pragma unroll
    for (int u = 0; u < IDS; ++u) {
        const int i = tid + AT * NS * u;
        if (i < n_rel) sm.rows[i] = key_code(kc, ki, (int32_t)j0 + i, ids[u]);
    }
    if (tid < ROPE_PAIRS) {
        double sn, cs;
        rope_sincos((double)ki.t * ifreq, &sn, &cs);
        sm.rsin[tid] = sn;
        sm.rcos[tid] = cs;
        sm.rsc[tid] = make_float2((float)sn, (float)cs);
    }
    if (NS > 1 && tid < NS) sm.sync[tid] = 0u;
    __syncthreads();

    // Scores are kept in log2 units: the softmax scale times log2(e) multiplies
    // the K row scales as they are staged and the rotated RoPE query here, and
    // the RoPE product's accumulator starts at the key's bias (0, or -inf for
    // an empty slot), so a score is one fma of the two products.
    const float sc2 = p.sm_scale * 1.4426950408889634f;
    // query operands (B of S^T = K Q^T): head `col` of this wave, dims 32c + 8g .. +8
    bf16x8 qrh[2], qrl[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const bf16x8 raw = qraw[c];
        bf16x8 hi, lo;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
            // float32 rotation: the hi + lo BF16 terms keep about 16 bits, far
            // below float32's rounding
            const int pr = (32 * c + 8 * g + i) >> 1;
            const float2 t = sm.rsc[pr];
            const float x = (float)raw[i], y = (float)raw[i + 1];
            const float rx = (x * t.y - y * t.x) * sc2, ry = (x * t.x + y * t.y) * sc2;
            hi[i] = (__bf16)rx;
            hi[i + 1] = (__bf16)ry;
            lo[i] = (__bf16)(rx - (float)hi[i]);
            lo[i + 1] = (__bf16)(ry - (float)hi[i + 1]);
        }
        qrh[c] = hi;
        qrl[c] = lo;
    }
    // The running max starts at a finite floor far below any logit, so that
    // exp2(s - mrun) is 0 for an empty slot (s = -inf) with no test.
    float mrun = -1e30f, lrun = 0.f;
    v4f O[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) O[i] = (v4f){0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    // two-stage pipeline: tile t+2 is loaded while tile t is staged and computed
    const int n_tiles = (n_rel + TK - 1) / TK;
    // Two tiles' loads are in flight per stream (a tile past the split's end
    // loads nothing and is staged empty), and the loop is unrolled by two, so
    // the wait before staging tile t only covers tile t's loads and tile t+1's
    // stay in flight.
    auto compute = [&](const TileBuf &tb) {
        if (!active) return;
        // per-key scales of this lane's eight keys (4g..4g+3 and 16+4g..), read as vectors
        v4f ks[2], kb[2], vs[2];
#pragma unroll
        for (int st = 0; st < 2; ++st) {
            ks[st] = *(const v4f *)&tb.ksc[16 * st + 4 * g];
            kb[st] = *(const v4f *)&tb.kbias[16 * st + 4 * g];
            vs[st] = *(const v4f *)&tb.vsc[16 * st + 4 * g];
        }
        // the two key halves as independent MFMA chains
        v4f an[2] = {zero, zero}, ar[2] = {kb[0], kb[1]};
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int st = 0; st < 2; ++st)
                an[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    ld16(&tb.kb[(16 * st + col) * KB_LD + 8 * g + 32 * c]), qn[c], an[st], 0, 0, 0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int st = 0; st < 2; ++st) {
                const bf16x8 a = ld16(&tb.kb[(16 * st + col) * KB_LD + 8 * g + MDN + 32 * c]);
                ar[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qrh[c], ar[st], 0, 0, 0);
                ar[st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qrl[c], ar[st], 0, 0, 0);
            }
        // an empty slot has a zero K row, a zero scale and bias -inf
        float s[2][4];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) s[st][j] = __builtin_fmaf(an[st][j], ks[st][j], ar[st][j]);
        float mx = s[0][0];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, s[st][j]);
        mx = swap32_max(swap16_max(mx));
        // raise the running max (and rescale) only when this tile exceeds it by the slack
        if (__builtin_amdgcn_ballot_w64(mx > mrun + RESCALE_SLACK)) {
            const float mn = __builtin_fmaxf(mrun, mx);
            const float c = __builtin_amdgcn_exp2f(mrun - mn);
            lrun *= c;
#pragma unroll
            for (int i = 0; i < 12; ++i) O[i] *= c;
            mrun = mn;
        }
        float pr[2][4], psum = 0.f;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pr[st][j] = __builtin_amdgcn_exp2f(s[st][j] - mrun);
                psum += pr[st][j];
            }
        lrun += swap32_sum(swap16_sum(psum));
        // P as two BF16 terms (hi + lo): one BF16 alone would cost 2^-9 of the
        // largest output element, which outliers in V turn into a visible error.
        // (pairs of values per conversion instruction)
        bf16x8 pnh, pnl, pbh, pbl;
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                const int e = 4 * st + j;
                split_bf16x2(pr[st][j] * vs[st][j], pr[st][j + 1] * vs[st][j + 1], pnh, pnl, e);
                split_bf16x2(pr[st][j], pr[st][j + 1], pbh, pbl, e);
            }
#pragma unroll
        for (int dt = 0; dt < 12; ++dt) {
            const bf16x8 a = vt_operand(tb, dt, g, col);
            O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dt < 8 ? pnh : pbh, O[dt], 0, 0, 0);
            O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dt < 8 ? pnl : pbl, O[dt], 0, 0, 0);
        }
    };
    // stream s: tiles s + NS i; every stream runs the same number of rounds
    // (a round past its last tile stages an empty tile and skips the compute)
    const int n_rounds = (n_tiles + NS - 1) / NS;
    // The workgroup holding the appended key encodes the row while the first
    // tiles are in flight (the barrier before the first staging publishes it).
    int cur = -1;
    if (app_here) {
        const int c = (int)(n_keys - 1 - j0);
        if (sm.rows[c] >= 0) cur = c;
    }
    // three waves split the encoding: the no-RoPE codes of K (the last
    // wave) and of V (the one before), and both RoPE pairs (the third last)
    if (cur >= 0 && aw < 3) {
        const int64_t row = sm.rows[cur] & (WIN_BIT - 1);
        const uint32_t raw = araw;
        if (aw < 2) {
            const bool isk = aw == 0;
            const KvView &st = isk ? p.wk : p.wv;
            uint8_t c0, c1;
            const float sc = e4m3_group128(bf16_decode((uint16_t)raw), bf16_decode((uint16_t)(raw >> 16)), &c0, &c1);
            const uint16_t cc = (uint16_t)(c0 | (c1 << 8));
            ((uint16_t *)(isk ? sm.app.kc : sm.app.vc))[lane] = cc;
            ((uint16_t *)(st.nope + b * st.nope_bs + row * st.nope_rs))[lane] = cc;
            if (lane == 0) {
                *(isk ? &sm.app.ksc : &sm.app.vsc) = sc;
                *(float *)(st.scale + b * st.scale_bs + row * st.scale_rs) = sc;
            }
        } else {
            // K's pair rotated at t (lanes 0..31), V's as it is (lanes 32..63)
            const int lr = lane & 31;
            const bool isk = lane < 32;
            uint32_t bits;
            if (isk) {
                double xr, yr;
                rope_rotate((double)bf16_decode((uint16_t)raw), (double)bf16_decode((uint16_t)(raw >> 16)),
                            sm.rsin[lr], sm.rcos[lr], &xr, &yr);
                bits = (uint32_t)bf16_encode((float)xr) | ((uint32_t)bf16_encode((float)yr) << 16);
            } else {
                bits = (uint32_t)bf16_encode(bf16_decode((uint16_t)raw)) |
                       ((uint32_t)bf16_encode(bf16_decode((uint16_t)(raw >> 16))) << 16);
            }
            ((uint32_t *)(isk ? sm.app.kr : sm.app.vr))[lr] = bits;
            const char *rp = isk ? p.wk.rope + b * p.wk.rope_bs + row * p.wk.rope_rs
                                 : p.wv.rope + b * p.wv.rope_bs + row * p.wv.rope_rs;
            ((uint32_t *)rp)[lr] = bits;
        }
    }
    // Double-buffered rounds with one barrier each: round r computes the
    // stream's tile r from one buffer while its tile r + 1 is staged into the
    // other (whose loads were issued a round earlier), and issues the loads of
    // tile r + 2 into the register set that staging freed.
    TileBuf &b0 = sm.tb[stream][0], &b1 = sm.tb[stream][1];
    // With two streams each round synchronises the stream's own four waves
    // (its tiles and buffers are its own): an LDS counter per stream that
    // every wave adds one to once its LDS stores are done, then waits for
    // (a bounded wait: every wave leaves it), so that one stream's late tile
    // does not hold the other back.
    uint32_t sync_gen = 0;
    auto round_sync = [&]() {
        if (NS == 1) {
            __syncthreads();
            return;
        }
        sync_gen += AT / 64;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this wave's LDS stores are done
        asm volatile("" ::: "memory");
        if (lane == 0) __hip_atomic_fetch_add(&sm.sync[stream], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        for (int spin = 0; spin < (1 << 16); ++spin) {
            if (__hip_atomic_load(&sm.sync[stream], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= sync_gen) break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    };
    __syncthreads();  // the resolved rows and the appended row are published
    stage_tile(RA, sm.rows, b0, stream * TK, n_rel, tids, sm.app, cur, sc2);
    load_tile<NT>(lsrc, sm.rows, (stream + 2 * NS) * TK, n_rel, RA, tids);
    round_sync();
    // The loop runs whole pairs of rounds and has no exit but its own test:
    // an exit from inside would join the loop's paths in one block, where the
    // compiler has to assume that the tile staged first is the newest load
    // and waits for every load in flight. The last one or two rounds follow.
    int i = 0;
    for (; i + 2 < n_rounds; i += 2) {
        const int ta = stream + NS * i, tb_ = stream + NS * (i + 1);
        if (ta < n_tiles) compute(b0);
        stage_tile(RB, sm.rows, b1, tb_ * TK, n_rel, tids, sm.app, cur, sc2);
        load_tile<NT>(lsrc, sm.rows, (tb_ + 2 * NS) * TK, n_rel, RB, tids);
        round_sync();
        if (tb_ < n_tiles) compute(b1);
        stage_tile(RA, sm.rows, b0, (ta + 2 * NS) * TK, n_rel, tids, sm.app, cur, sc2);
        load_tile<NT>(lsrc, sm.rows, (ta + 4 * NS) * TK, n_rel, RA, tids);
        round_sync();
    }
    if (i < n_rounds) {  // uniform
        const int ta = stream + NS * i, tb_ = stream + NS * (i + 1);
        if (ta < n_tiles) compute(b0);
        if (i + 1 < n_rounds) {
            stage_tile(RB, sm.rows, b1, tb_ * TK, n_rel, tids, sm.app, cur, sc2);
            round_sync();
            if (tb_ < n_tiles) compute(b1);
        }
    }
    if (NS > 1) {
        // the other streams hand their (max, sum, O) to stream 0 through the tile buffers
        __syncthreads();
        float *xo = (float *)&sm.tb[0][0];
        static_assert(sizeof(TileBuf) * 2 * NS >= sizeof(float) * AT * 48 * (NS - 1), "exchange fits the tile buffers");
        if (stream > 0 && active) {
            const int base = (stream - 1) * AT * 48;
#pragma unroll
            for (int dt = 0; dt < 12; ++dt) *(v4f *)&xo[base + (dt * AT + tids) * 4] = O[dt];
            sm.xml[2 * tids] = mrun;
            sm.xml[2 * tids + 1] = lrun;
        }
        __syncthreads();
        if (stream > 0) return;
        if (active) {
#pragma unroll
            for (int os = 1; os < NS; ++os) {
                const int base = (os - 1) * AT * 48;
                const float m1 = sm.xml[2 * tids], l1 = sm.xml[2 * tids + 1];
                const float mn = __builtin_fmaxf(mrun, m1);
                const float c0 = __builtin_amdgcn_exp2f(mrun - mn);
                const float c1 = __builtin_amdgcn_exp2f(m1 - mn);
#pragma unroll
                for (int dt = 0; dt < 12; ++dt) O[dt] = O[dt] * c0 + *(const v4f *)&xo[base + (dt * AT + tids) * 4] * c1;
                lrun = lrun * c0 + l1 * c1;
                mrun = mn;
            }
        }
    }
    if (!active) return;
    // epilogue: lane holds O^T[16dt + 4g + j][head]
    if (p.n_split == 1) {
        const float inv = lrun > 0.f ? 1.f / lrun : 0.f;
        if (p.o_bf16) {
            __bf16 *op = (__bf16 *)p.o + ((size_t)q * H + head) * MD;
#pragma unroll
            for (int dt = 0; dt < 12; ++dt) {
                bf16x2 a = {(__bf16)(O[dt][0] * inv), (__bf16)(O[dt][1] * inv)};
                bf16x2 c = {(__bf16)(O[dt][2] * inv), (__bf16)(O[dt][3] * inv)};
                v2u pk = {__builtin_bit_cast(unsigned, a), __builtin_bit_cast(unsigned, c)};
                *(v2u *)(op + 16 * dt + 4 * g) = pk;
            }
        } else {
            float *op = (float *)p.o + ((size_t)q * H + head) * MD;
#pragma unroll
            for (int dt = 0; dt < 12; ++dt) *(v4f *)(op + 16 * dt + 4 * g) = O[dt] * inv;
        }
        if (g == 0 && p.lse)
            p.lse[(size_t)q * H + head] = lrun > 0.f ? (mrun + log2f(lrun)) * 0.6931471805599453f : -__builtin_inff();
    } else {
        // Non-temporal stores: the partials of all splits (7-10 MB per decode
        // launch) are read once, by the combine, mostly on other XCDs. Written
        // as ordinary lines they made the decode step about 1.5 us slower
        // (measured; the likely cause is their write-back from this XCD's L2
        // at the kernel's end).
        const size_t base = ((size_t)q * p.n_split + split) * H + head;
        float *po = p.part_o + base * MD;
#pragma unroll
        for (int dt = 0; dt < 12; ++dt) __builtin_nontemporal_store(O[dt], (v4f *)(po + 16 * dt + 4 * g));
        if (g == 0) {
            __builtin_nontemporal_store(mrun, &p.part_ml[base * 2]);
            __builtin_nontemporal_store(lrun, &p.part_ml[base * 2 + 1]);
        }
    }
}

// -------------------------------------------------------------- combine ----

constexpr int MAX_SPLIT = 1024;
constexpr int CMB_G = 4;                 // threads sharing one output dim (few query-head pairs)
constexpr int CMB_MANY = 512;            // query-head pairs from which one thread per dim is used
constexpr int CMB_CHUNK = 32;            // splits a combine thread loads at once

// Merge the splits of one (query, head). G threads share output dim d:
// thread group gi takes splits gi, gi + G, ...; every partial output a
// thread needs (up to CMB_CHUNK) is loaded before the split weights are known,
// so one memory round trip covers the partials and the (max, sum) pairs. The
// groups' sums are added in a fixed order (deterministic).
template <int OUT_BF16, int G>
__global__ __launch_bounds__(G * 192) void attn_combine_kernel(AttnPlan p) {
    constexpr int CMB_T = G * 192;
    constexpr int NK = (MAX_SPLIT + CMB_T - 1) / CMB_T;  // (max, sum) pairs a thread loads
    __shared__ float wgt[MAX_SPLIT];
    __shared__ float red[2][CMB_T / 64];
    __shared__ float part[G > 1 ? G - 1 : 1][192];
    const int q = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int D = p.D, H = p.H, S = p.n_split;
    const int d = tid % 192, gi = tid / 192;
    const size_t base = (size_t)q * S * H;
    const size_t stride = (size_t)H * D;
    const bool own = d < D;
    const float *po = p.part_o + (base + h) * D + (own ? d : 0);
    float v[CMB_CHUNK];
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; ++i) {
        const int sp = gi + G * i;
        v[i] = (own && sp < S) ? __builtin_nontemporal_load(&po[(size_t)sp * stride]) : 0.f;
    }
    float2 ml[NK];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int sp = tid + CMB_T * k;
        ml[k] = sp < S ? ld_ml(&p.part_ml[((base + (size_t)sp * H) + h) * 2]) : make_float2(-__builtin_inff(), 0.f);
        mloc = __builtin_fmaxf(mloc, ml[k].x);
    }
    mloc = wave_max(mloc);
    if (lane == 0) red[0][wave] = mloc;
    __syncthreads();
    float M = red[0][0];
#pragma unroll
    for (int w = 1; w < CMB_T / 64; ++w) M = __builtin_fmaxf(M, red[0][w]);
    float lloc = 0.f;
#pragma unroll
    for (int k = 0; k < NK; ++k) {
        const int sp = tid + CMB_T * k;
        if (sp < S) {
            const float w = M == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(ml[k].x - M);
            wgt[sp] = w;
            lloc += w * ml[k].y;
        }
    }
    lloc = wave_sum(lloc);
    if (lane == 0) red[1][wave] = lloc;
    __syncthreads();
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < CMB_T / 64; ++w) L += red[1][w];
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < CMB_CHUNK; ++i) {
        const int sp = gi + G * i;
        if (sp < S) acc += v[i] * wgt[sp];
    }
    for (int s0 = G * CMB_CHUNK; s0 < S; s0 += G * CMB_CHUNK) {  // more than 128 splits
#pragma unroll
        for (int i = 0; i < CMB_CHUNK; ++i) {
            const int sp = s0 + gi + G * i;
            v[i] = (own && sp < S) ? __builtin_nontemporal_load(&po[(size_t)sp * stride]) : 0.f;
        }
#pragma unroll
        for (int i = 0; i < CMB_CHUNK; ++i) {
            const int sp = s0 + gi + G * i;
            if (sp < S) acc += v[i] * wgt[sp];
        }
    }
    if (gi > 0) part[gi - 1][d] = acc;
    __syncthreads();
    if (gi == 0 && own) {
#pragma unroll
        for (int k = 0; k < G - 1; ++k) acc += part[k][d];
        const float o = L > 0.f ? acc / L : 0.f;
        if (OUT_BF16) ((__bf16 *)p.o)[((size_t)q * H + h) * D + d] = (__bf16)o;
        else ((float *)p.o)[((size_t)q * H + h) * D + d] = o;
    }
    if (tid == 0 && p.lse)
        p.lse[(size_t)q * H + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -__builtin_inff();
}

// Merge of at most 64 splits: thread d of a (query, head) workgroup sums
// output dim d over the splits itself, and every wave reduces the splits'
// (max, sum) pairs on its own (lane j holds split j), so the merge needs no
// LDS and no barrier. NS: splits loaded per thread, a multiple of 16 at or
// above the split count (the surplus loads repeat the last split and get
// weight zero, so that every load and product is unconditional). The
// splits are added in split order (deterministic).
template <int OUT_BF16, int NS>
__global__ __launch_bounds__(192) void attn_combine_w_kernel(AttnPlan p) {
    static_assert(NS % 16 == 0 && NS <= 64, "one lane per split");
    const int q = blockIdx.x, h = blockIdx.y, d = threadIdx.x, lane = d & 63;
    const int D = p.D, H = p.H, S = p.n_split;
    const size_t base = (size_t)q * S * H;
    const size_t stride = (size_t)H * D;
    const bool own = d < D;
    const int dd = own ? d : 0;
    // every load in one batch: the partials of dim d (split i's row is a
    // scalar address stepped by stride), then lane j's (max, sum) pair
    const float *row = p.part_o + (base + h) * D;
    float v[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        v[i] = __builtin_nontemporal_load(&row[dd]);
        row += i + 1 < S ? stride : 0;
    }
    const int j = lane < S ? lane : S - 1;
    const float2 ml = ld_ml(&p.part_ml[((base + (size_t)j * H) + h) * 2]);
    __builtin_amdgcn_sched_barrier(0);
    const float mj = lane < S ? __builtin_fmaxf(-__builtin_inff(), ml.x) : -__builtin_inff();
    const float M = wave_max_dpp(mj);
    const float wj = (lane < S && M != -__builtin_inff()) ? __builtin_amdgcn_exp2f(ml.x - M) : 0.f;
    const float L = wave_sum_dpp(wj * (lane < S ? ml.y : 0.f));
    // splits past S repeat split S - 1's partial with weight zero (a finite
    // partial adds zero; a NaN one makes the output NaN either way)
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NS; ++i) acc = __builtin_fmaf(v[i], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wj), i)), acc);
    if (own) {
        const float o = L > 0.f ? acc / L : 0.f;
        if (OUT_BF16) ((__bf16 *)p.o)[((size_t)q * H + h) * D + d] = (__bf16)o;
        else ((float *)p.o)[((size_t)q * H + h) * D + d] = o;
    }
    if (d == 0 && p.lse)
        p.lse[(size_t)q * H + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -__builtin_inff();
}

template <int NS>
static void launch_combine_w(const AttnPlan &p, hipStream_t s) {
    if (p.o_bf16) hipLaunchKernelGGL((attn_combine_w_kernel<1, NS>), dim3(p.Q, p.H), dim3(192), 0, s, p);
    else hipLaunchKernelGGL((attn_combine_w_kernel<0, NS>), dim3(p.Q, p.H), dim3(192), 0, s, p);
}

template <int NS, bool NT>
static void launch_mx(const AttnPlan &p, const dim3 &grid, hipStream_t s) {
    switch (p.H / 16) {
        case 1: hipLaunchKernelGGL((attn_mx_kernel<1, NS, NT>), grid, dim3(NS * AT), 0, s, p); break;
        case 2: hipLaunchKernelGGL((attn_mx_kernel<2, NS, NT>), grid, dim3(NS * AT), 0, s, p); break;
        case 3: hipLaunchKernelGGL((attn_mx_kernel<3, NS, NT>), grid, dim3(NS * AT), 0, s, p); break;
        default: hipLaunchKernelGGL((attn_mx_kernel<4, NS, NT>), grid, dim3(NS * AT), 0, s, p); break;
    }
}

static void launch_attn_slice(const AttnPlan &p, int nq, hipStream_t s) {
    const dim3 grid(p.n_split, nq);
    if (p.ek.fmt == 0 && p.wk.fmt == 0) {
        size_t lds = (size_t)(p.H * p.D + 2 * TK * p.D + p.H * TK + 3 * p.H) * 4;
        hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(AT), lds, s, p);
    } else if (p.n_streams == 2) {
        if (p.Tq == 1) launch_mx<2, true>(p, grid, s);
        else launch_mx<2, false>(p, grid, s);
    } else {
        if (p.Tq == 1) launch_mx<1, true>(p, grid, s);
        else launch_mx<1, false>(p, grid, s);
    }
}

hipError_t launch_attn(const AttnPlan &plan, hipStream_t s) {
    AttnPlan p = plan;
    KeyConsts &kc = p.kc;
    kc.W = p.W;
    kc.ring = (int32_t)p.wk.ring;
    kc.wrows = (int32_t)p.wk.rows;
    kc.erows = p.has_ent ? (int32_t)p.ek.rows : 0;
    int64_t cap = 0;
    if (p.has_ent) {
        cap = p.sparse ? p.k : p.ek.rows;
        if (!p.sparse && p.n_override >= 0 && p.n_override < cap) cap = p.n_override;
    }
    kc.cap = (int32_t)cap;
    uint32_t m_sh = 0, r_sh = 0;
    div_consts(p.m, &kc.m_mul, &m_sh);
    kc.r_mul = 0;
    if (kc.ring > 0) div_consts(kc.ring, &kc.r_mul, &r_sh);
    kc.misc = (p.sparse ? 1u : 0u) | (m_sh << 8) | (r_sh << 16);
    kc.m = p.m;
    for (int q0 = 0; q0 < p.Q; q0 += MAX_GRID_Y) {
        AttnPlan ps = p;
        ps.q_base = q0;
        launch_attn_slice(ps, p.Q - q0 < MAX_GRID_Y ? p.Q - q0 : MAX_GRID_Y, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    // many query-head pairs (several tokens per sequence): one thread per output dim
    // sums every split; few pairs (one decode token): CMB_G threads share a dim
    const bool many = (int64_t)p.Q * p.H >= CMB_MANY;
    if (!many && p.n_split <= 64) {
        switch ((p.n_split + 15) / 16) {
            case 1: launch_combine_w<16>(p, s); break;
            case 2: launch_combine_w<32>(p, s); break;
            case 3: launch_combine_w<48>(p, s); break;
            default: launch_combine_w<64>(p, s); break;
        }
        return hipGetLastError();
    }
    if (p.o_bf16) {
        if (many) hipLaunchKernelGGL((attn_combine_kernel<1, 1>), dim3(p.Q, p.H), dim3(192), 0, s, p);
        else hipLaunchKernelGGL((attn_combine_kernel<1, CMB_G>), dim3(p.Q, p.H), dim3(CMB_G * 192), 0, s, p);
    } else {
        if (many) hipLaunchKernelGGL((attn_combine_kernel<0, 1>), dim3(p.Q, p.H), dim3(192), 0, s, p);
        else hipLaunchKernelGGL((attn_combine_kernel<0, CMB_G>), dim3(p.Q, p.H), dim3(CMB_G * 192), 0, s, p);
    }
    return hipGetLastError();
}

__global__ void fill_zero_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t s) {
    const size_t n = bytes / 4;
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t *)ptr, n);
    return hipGetLastError();
}

}  // namespace v4a
