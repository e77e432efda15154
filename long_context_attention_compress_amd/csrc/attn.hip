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
//    to match), V is staged transposed in LDS, and the V row scale is folded
//    into P for the E4M3 dims; P also goes in as two BF16 terms (hi + lo).
//  * All 64 heads of a workgroup share each staged K/V tile.
//  * The raw bytes of every tile of the split are loaded into registers before
//    any is used, so one HBM round trip covers the whole split.

#include "common.hpp"

namespace v4a {

constexpr int AT = 256;
constexpr int TK = 32;  // keys per tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v2u __attribute__((ext_vector_type(2)));

struct KeyInfo {
    int64_t n_list;  // entries in the list
    int64_t n_win;   // window rows
    int64_t t;
};

__device__ __forceinline__ KeyInfo key_info(const AttnPlan &p, int q) {
    KeyInfo ki;
    ki.t = p.q_pos[q];
    if (ki.t < 0) {
        ki.n_list = 0;
        ki.n_win = 0;
        return ki;
    }
    ki.n_win = ki.t + 1 < p.W ? ki.t + 1 : p.W;
    if (!p.has_ent) ki.n_list = 0;
    else if (p.sparse) ki.n_list = p.k;
    else {
        int64_t n = (ki.t + 1) / p.m;
        if (n > p.ek.rows) n = p.ek.rows;
        if (p.n_override >= 0 && n > p.n_override) n = p.n_override;
        ki.n_list = n;
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
    const int q = blockIdx.y, split = blockIdx.x;
    const int b = q / p.Tq;
    const KeyInfo ki = key_info(p, q);
    const float *qin = (const float *)p.q + (size_t)q * H * D;
    const int Dn = D - ROPE_DIM;
    for (int i = tid; i < H * D; i += AT) {
        const int h = i / D, d = i % D;
        float v = qin[i];
        if (d >= Dn) {
            const int r = d - Dn, pr = r >> 1;
            double sn, cs;
            sincos((double)ki.t * p.inv_freq[pr], &sn, &cs);
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
constexpr int KB_LD = MD + 8;   // bf16 elements per staged K row (padded)
constexpr int VT_LD = TK + 8;   // bf16 elements per staged V^T row (padded)
constexpr int PF = 4;           // tiles whose raw bytes are loaded together

struct MxSmem {
    __bf16 kb[TK * KB_LD];
    __bf16 vt[MD * VT_LD];
    float ksc[TK];
    float vsc[TK];
    int kval[TK];
};

struct TileRegs {
    v4i k[2], v[2];
    float sc;
    int row[2];
    int win[2];
};

__device__ __forceinline__ void load_tile(const AttnPlan &p, int q, int b, const KeyInfo &ki, int64_t jt, int64_t j1,
                                          TileRegs &R) {
    const int tid = threadIdx.x;
    const int part = tid & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (tid >> 4) + 16 * h;
        bool win = false;
        const int64_t row = (jt + r < j1) ? key_row(p, q, ki, jt + r, &win) : -1;
        R.row[h] = (int)(row >= 0);
        R.win[h] = win;
        v4i kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
        if (row >= 0) {
            const KvView &K = win ? p.wk : p.ek;
            const KvView &V = win ? p.wv : p.ev;
            const char *kp = part < 8 ? K.nope + b * K.nope_bs + row * K.nope_rs + 16 * part
                                      : K.rope + b * K.rope_bs + row * K.rope_rs + 16 * (part - 8);
            const char *vp = part < 8 ? V.nope + b * V.nope_bs + row * V.nope_rs + 16 * part
                                      : V.rope + b * V.rope_bs + row * V.rope_rs + 16 * (part - 8);
            kx = __builtin_nontemporal_load((const v4i *)kp);
            vx = __builtin_nontemporal_load((const v4i *)vp);
        }
        R.k[h] = kx;
        R.v[h] = vx;
    }
    // scales: threads 0..31 -> K scale of key tid, 32..63 -> V scale of key tid-32
    R.sc = 0.f;
    if (tid < 2 * TK) {
        const int r = tid & (TK - 1);
        bool win = false;
        const int64_t row = (jt + r < j1) ? key_row(p, q, ki, jt + r, &win) : -1;
        if (row >= 0) {
            const KvView &S = (tid < TK) ? (win ? p.wk : p.ek) : (win ? p.wv : p.ev);
            R.sc = *(const float *)(S.scale + b * S.scale_bs + row * S.scale_rs);
        }
    }
}

template <bool HI>
__device__ __forceinline__ unsigned fp8x2_to_bf16x2(unsigned w) {
    bf16x2 v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
    return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ void stage_tile(const TileRegs &R, MxSmem &sm) {
    const int tid = threadIdx.x;
    const int part = tid & 15;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = (tid >> 4) + 16 * h;
        if (part < 8) {
            // 16 E4M3 codes -> 16 BF16 (exact)
            v4i c = R.k[h];
            v4i lo, hi;
            lo[0] = fp8x2_to_bf16x2<false>(c[0]);
            lo[1] = fp8x2_to_bf16x2<true>(c[0]);
            lo[2] = fp8x2_to_bf16x2<false>(c[1]);
            lo[3] = fp8x2_to_bf16x2<true>(c[1]);
            hi[0] = fp8x2_to_bf16x2<false>(c[2]);
            hi[1] = fp8x2_to_bf16x2<true>(c[2]);
            hi[2] = fp8x2_to_bf16x2<false>(c[3]);
            hi[3] = fp8x2_to_bf16x2<true>(c[3]);
            *(v4i *)&sm.kb[r * KB_LD + 16 * part] = lo;
            *(v4i *)&sm.kb[r * KB_LD + 16 * part + 8] = hi;
            v4i cv = R.v[h];
            unsigned u[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                u[2 * i] = fp8x2_to_bf16x2<false>(cv[i]);
                u[2 * i + 1] = fp8x2_to_bf16x2<true>(cv[i]);
            }
            unsigned short *vt = (unsigned short *)sm.vt;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                vt[(16 * part + 2 * i) * VT_LD + r] = (unsigned short)(u[i] & 0xFFFF);
                vt[(16 * part + 2 * i + 1) * VT_LD + r] = (unsigned short)(u[i] >> 16);
            }
        } else {
            *(v4i *)&sm.kb[r * KB_LD + MDN + 8 * (part - 8)] = R.k[h];
            v4i cv = R.v[h];
            unsigned short *vt = (unsigned short *)sm.vt;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                vt[(MDN + 8 * (part - 8) + 2 * i) * VT_LD + r] = (unsigned short)((unsigned)cv[i] & 0xFFFF);
                vt[(MDN + 8 * (part - 8) + 2 * i + 1) * VT_LD + r] = (unsigned short)((unsigned)cv[i] >> 16);
            }
        }
    }
    if (tid < TK) {
        sm.ksc[tid] = R.sc;
    } else if (tid < 2 * TK) {
        sm.vsc[tid - TK] = R.sc;
    }
    // validity: thread with part == 0 owns rows (tid>>4) and 16+(tid>>4)
    if (part == 0) {
        sm.kval[(tid >> 4)] = R.row[0];
        sm.kval[16 + (tid >> 4)] = R.row[1];
    }
}

__device__ __forceinline__ bf16x8 lds8(const __bf16 *p) { return *(const bf16x8 *)p; }
__device__ __forceinline__ bf16x8 lds4x2(const __bf16 *a, const __bf16 *b) {
    v2u x = *(const v2u *)a, y = *(const v2u *)b;
    v4i r = {(int)x[0], (int)x[1], (int)y[0], (int)y[1]};
    return __builtin_bit_cast(bf16x8, r);
}

template <int NW>
__global__ __launch_bounds__(AT) void attn_mx_kernel(AttnPlan p) {
    __shared__ MxSmem sm;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int q = blockIdx.y, split = blockIdx.x;
    const int b = q / p.Tq;
    const KeyInfo ki = key_info(p, q);
    const int H = p.H;
    const bool active = wave < NW;
    const int head = 16 * wave + col;

    // query operands (B of S^T = K Q^T): head `col` of this wave, dims 32c + 8g .. +8
    bf16x8 qn[4], qrh[2], qrl[2];
    {
        const int hh = active ? head : 0;
        const __bf16 *qp = (const __bf16 *)p.q + ((size_t)q * H + hh) * MD;
#pragma unroll
        for (int c = 0; c < 4; ++c) qn[c] = lds8(qp + 32 * c + 8 * g);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8 raw = lds8(qp + MDN + 32 * c + 8 * g);
            bf16x8 hi, lo;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const int pr = (32 * c + 8 * g + i) >> 1;
                double sn, cs;
                sincos((double)ki.t * p.inv_freq[pr], &sn, &cs);
                const double x = (double)(float)raw[i], y = (double)(float)raw[i + 1];
                const float rx = (float)(x * cs - y * sn), ry = (float)(x * sn + y * cs);
                hi[i] = (__bf16)rx;
                hi[i + 1] = (__bf16)ry;
                lo[i] = (__bf16)(rx - (float)hi[i]);
                lo[i + 1] = (__bf16)(ry - (float)hi[i + 1]);
            }
            qrh[c] = hi;
            qrl[c] = lo;
        }
    }
    const float sc2 = p.sm_scale * 1.4426950408889634f;
    float mrun = -__builtin_inff(), lrun = 0.f;
    v4f O[12];
#pragma unroll
    for (int i = 0; i < 12; ++i) O[i] = (v4f){0.f, 0.f, 0.f, 0.f};

    const int64_t n_keys = ki.n_list + ki.n_win;
    const int64_t j0 = (int64_t)split * p.keys_per_split;
    const int64_t j1 = j0 + p.keys_per_split < n_keys ? j0 + p.keys_per_split : n_keys;
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    for (int64_t jg = j0; jg < j1; jg += PF * TK) {
        TileRegs R[PF];
#pragma unroll
        for (int u = 0; u < PF; ++u)
            if (jg + u * TK < j1) load_tile(p, q, b, ki, jg + u * TK, j1, R[u]);
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            if (jg + u * TK >= j1) break;
            __syncthreads();
            stage_tile(R[u], sm);
            __syncthreads();
            if (active) {
                float s[2][4];
#pragma unroll
                for (int st = 0; st < 2; ++st) {
                    v4f an = zero, ar = zero;
                    const __bf16 *krow = &sm.kb[(16 * st + col) * KB_LD + 8 * g];
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        an = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds8(krow + 32 * c), qn[c], an, 0, 0, 0);
#pragma unroll
                    for (int c = 0; c < 2; ++c) {
                        bf16x8 a = lds8(krow + MDN + 32 * c);
                        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qrh[c], ar, 0, 0, 0);
                        ar = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qrl[c], ar, 0, 0, 0);
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = 16 * st + 4 * g + j;
                        s[st][j] = sm.kval[key] ? (an[j] * sm.ksc[key] + ar[j]) * sc2 : -__builtin_inff();
                    }
                }
                float mx = s[0][0];
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) mx = __builtin_fmaxf(mx, s[st][j]);
                mx = __builtin_fmaxf(mx, __shfl_xor(mx, 16, 64));
                mx = __builtin_fmaxf(mx, __shfl_xor(mx, 32, 64));
                const float mn = __builtin_fmaxf(mrun, mx);
                float c = 1.f, psum = 0.f;
                float pr[2][4];
                if (mn != -__builtin_inff()) {
                    c = exp2f(mrun - mn);
#pragma unroll
                    for (int st = 0; st < 2; ++st)
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            pr[st][j] = exp2f(s[st][j] - mn);
                            psum += pr[st][j];
                        }
                } else {
#pragma unroll
                    for (int st = 0; st < 2; ++st)
#pragma unroll
                        for (int j = 0; j < 4; ++j) pr[st][j] = 0.f;
                }
                psum += __shfl_xor(psum, 16, 64);
                psum += __shfl_xor(psum, 32, 64);
                lrun = lrun * c + psum;
                mrun = mn;
#pragma unroll
                for (int i = 0; i < 12; ++i) O[i] *= c;
                // P as two BF16 terms (hi + lo): one BF16 alone would cost 2^-9 of the
                // largest output element, which outliers in V turn into a visible error.
                bf16x8 pnh, pnl, pbh, pbl;
#pragma unroll
                for (int st = 0; st < 2; ++st)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int key = 16 * st + 4 * g + j;
                        const float xn = pr[st][j] * sm.vsc[key], xb = pr[st][j];
                        pnh[4 * st + j] = (__bf16)xn;
                        pnl[4 * st + j] = (__bf16)(xn - (float)pnh[4 * st + j]);
                        pbh[4 * st + j] = (__bf16)xb;
                        pbl[4 * st + j] = (__bf16)(xb - (float)pbh[4 * st + j]);
                    }
#pragma unroll
                for (int dt = 0; dt < 12; ++dt) {
                    const __bf16 *vr = &sm.vt[(16 * dt + col) * VT_LD];
                    bf16x8 a = lds4x2(vr + 4 * g, vr + 16 + 4 * g);
                    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dt < 8 ? pnh : pbh, O[dt], 0, 0, 0);
                    O[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, dt < 8 ? pnl : pbl, O[dt], 0, 0, 0);
                }
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
        const size_t base = ((size_t)q * p.n_split + split) * H + head;
        float *po = p.part_o + base * MD;
#pragma unroll
        for (int dt = 0; dt < 12; ++dt) *(v4f *)(po + 16 * dt + 4 * g) = O[dt];
        if (g == 0) {
            p.part_ml[base * 2] = mrun;
            p.part_ml[base * 2 + 1] = lrun;
        }
    }
}

// -------------------------------------------------------------- combine ----

template <int OUT_BF16>
__global__ void attn_combine_kernel(AttnPlan p) {
    const int q = blockIdx.x, h = blockIdx.y;
    const int D = p.D, H = p.H, S = p.n_split;
    const size_t base = (size_t)q * S * H;
    float M = -__builtin_inff();
    for (int s = 0; s < S; ++s) M = __builtin_fmaxf(M, p.part_ml[((base + (size_t)s * H) + h) * 2]);
    float L = 0.f;
    if (M != -__builtin_inff())
        for (int s = 0; s < S; ++s) {
            const size_t i = (base + (size_t)s * H) + h;
            L += p.part_ml[i * 2 + 1] * exp2f(p.part_ml[i * 2] - M);
        }
    for (int d = threadIdx.x; d < D; d += blockDim.x) {
        float o = 0.f;
        if (L > 0.f) {
            for (int s = 0; s < S; ++s) {
                const size_t i = (base + (size_t)s * H) + h;
                o += p.part_o[i * D + d] * exp2f(p.part_ml[i * 2] - M);
            }
            o /= L;
        }
        if (OUT_BF16) ((__bf16 *)p.o)[((size_t)q * H + h) * D + d] = (__bf16)o;
        else ((float *)p.o)[((size_t)q * H + h) * D + d] = o;
    }
    if (threadIdx.x == 0 && p.lse)
        p.lse[(size_t)q * H + h] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -__builtin_inff();
}

hipError_t launch_attn(const AttnPlan &p, hipStream_t s) {
    dim3 grid(p.n_split, p.Q);
    if (p.ek.fmt == 0 && p.wk.fmt == 0) {
        size_t lds = (size_t)(p.H * p.D + 2 * TK * p.D + p.H * TK + 3 * p.H) * 4;
        hipLaunchKernelGGL(attn_f32_kernel, grid, dim3(AT), lds, s, p);
    } else {
        switch (p.H / 16) {
            case 1: hipLaunchKernelGGL(attn_mx_kernel<1>, grid, dim3(AT), 0, s, p); break;
            case 2: hipLaunchKernelGGL(attn_mx_kernel<2>, grid, dim3(AT), 0, s, p); break;
            case 3: hipLaunchKernelGGL(attn_mx_kernel<3>, grid, dim3(AT), 0, s, p); break;
            default: hipLaunchKernelGGL(attn_mx_kernel<4>, grid, dim3(AT), 0, s, p); break;
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.n_split == 1) return e;
    if (p.o_bf16) hipLaunchKernelGGL(attn_combine_kernel<1>, dim3(p.Q, p.H), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(attn_combine_kernel<0>, dim3(p.Q, p.H), dim3(256), 0, s, p);
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
