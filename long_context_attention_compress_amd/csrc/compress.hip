// csa_compress: softmax-gated pooling of m raw tokens into one cache entry.
//
// [chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich nutzbar",
// section "Hybrid Attention: CSA und HCA"]: CSA compresses KV entries 4x along
// the sequence by softmax-gated pooling with a learned positional bias; HCA
// compresses 128x. [golem.de, "... Bei Deepseek V4 haben kleine Änderungen
// große Wirkung", section "Komprimierte Erinnerung für längere Kontexte"]: the
// last 64 values carry RoPE and stay BF16, the rest is FP8.
//
// Eight waves per (entry, batch element, output) for long blocks (an eighth
// of the tokens each), one wave per output in one workgroup for blocks of up
// to four tokens, and one wave per output for each two tokens of a chunk of
// window rows (m = 1); every lane holds pairs of adjacent elements of a row.
// The gate weights, the RoPE rotation and the weighted sum are evaluated in
// float64 and the entry is rounded to float32 before it is encoded, so every
// encoding decision (FP8 scale and codes, BF16 rounding, MX exponent and E2M1
// codes) is taken on a float32 value. That float64 work, not HBM, bounds these
// kernels; compression is a small share of decode time (one block per m
// tokens), so they keep the exact path.

#include "common.hpp"

namespace v4a {

constexpr int MAX_M = 1024;

template <int ACT>
__device__ __forceinline__ double load_act(const void *base, int64_t i) {
    if (ACT == 0) return (double)((const float *)base)[i];
    return (double)bf16_decode(((const uint16_t *)base)[i]);
}

__device__ __forceinline__ int64_t kv_row(const KvView &s, int64_t e) { return s.ring > 0 ? e % s.ring : e; }

// Where block j of batch element b comes from and goes to: `tok0` its first
// raw row (relative to the batch element's rows of the raw inputs), `first`
// the position of its first token, `entry` the entry it becomes. In block
// mode the block ends at the device position block_end[b]; the raw rows are a
// ring of t_new rows (a multiple of m), so the block's m rows are contiguous
// from row first % t_new. `ok` is false when nothing is to be written.
struct BlockGeo {
    bool ok;
    int64_t tok0, first, entry;
};
__device__ __forceinline__ BlockGeo block_geo(const CompressPlan &p, int j, int b, int m) {
    BlockGeo g;
    if (!p.block_end) {
        g.ok = true;
        g.tok0 = (int64_t)j * m;
        g.first = p.pos0 + g.tok0;
        g.entry = p.pos0 / m + j;
        return g;
    }
    const int64_t t = p.block_end[b];
    g.ok = t >= m - 1 && (t + 1) % m == 0;
    g.first = g.ok ? t + 1 - m : 0;
    g.tok0 = g.first % p.t_new;
    g.entry = g.first / m;
    // a linear store (or the indexer store) must hold the entry
    if ((p.has_kv && p.k.ring == 0 && (g.entry >= p.k.rows || g.entry >= p.v.rows)) ||
        (p.has_ik && g.entry >= p.ik.rows))
        g.ok = false;
    return g;
}

// Encode one float32 row held across the wave (nope dims lane + 64*i, rope
// pair `lane` for lanes < 32) into a KV store row.
__device__ void store_kv_row(const KvView &s, int b, int64_t row, const float *nope, int n_nope_it,
                             float rx, float ry) {
    const int lane = lane_id();
    const int Dn = s.dim - ROPE_DIM;
    if (s.fmt == 0) {
        float *dst = (float *)(s.f32 + b * s.f32_bs + row * s.f32_rs);
        for (int i = 0; i < n_nope_it; ++i) dst[lane + 64 * i] = nope[i];
        if (lane < ROPE_PAIRS) {
            dst[Dn + 2 * lane] = rx;
            dst[Dn + 2 * lane + 1] = ry;
        }
        return;
    }
    uint8_t *codes = (uint8_t *)(s.nope + b * s.nope_bs + row * s.nope_rs);
    float *scales = (float *)(s.scale + b * s.scale_bs + row * s.scale_rs);
    for (int g = 0; g < n_nope_it / 2; ++g) {  // groups of 128 dims = two lane iterations
        uint8_t c0, c1;
        const float sc = e4m3_group128(nope[2 * g], nope[2 * g + 1], &c0, &c1);
        codes[128 * g + lane] = c0;
        codes[128 * g + 64 + lane] = c1;
        if (lane == 0) scales[g] = sc;
    }
    if (lane < ROPE_PAIRS) {
        uint32_t *r = (uint32_t *)(s.rope + b * s.rope_bs + row * s.rope_rs);
        r[lane] = (uint32_t)bf16_encode(rx) | ((uint32_t)bf16_encode(ry) << 16);
    }
}

// Encode one pooled indexer value held by this lane (dimension d) into the
// indexer store; every lane of the wave calls it (MX blocks are 32 lanes).
__device__ __forceinline__ void store_ik_value(const IkView &s, int b, int64_t entry, int d, bool on, float x) {
    const int lane = lane_id();
    if (s.fmt == 0) {
        if (on) ((float *)(s.f32 + b * s.f32_bs + entry * s.f32_rs))[d] = x;
        return;
    }
    // MX block of 32 = one half of the wave
    bool bad = !__builtin_isfinite(x) && on;
    float a = on ? amax_acc(0.0f, x) : 0.0f;
    a = half_amax_bits(a);
    int nbad = __builtin_popcountll(__ballot(bad) & ((lane < 32) ? 0xFFFFFFFFull : 0xFFFFFFFF00000000ull));
    uint32_t code = 0;
    int E = 0;
    if (nbad == 0) {
        E = mx_exponent(a);
        code = e2m1_encode(__builtin_ldexpf(x, -E));
    }
    uint32_t nb = __shfl_down(code, 1, 64);
    if (on && (lane & 1) == 0)
        ((uint8_t *)(s.e2m1 + b * s.e2m1_bs + entry * s.e2m1_rs))[d >> 1] = (uint8_t)(code | (nb << 4));
    if (on && (lane & 31) == 0)
        ((uint8_t *)(s.e8m0 + b * s.e8m0_bs + entry * s.e8m0_rs))[d >> 5] = nbad ? 0xFF : (uint8_t)(E + 127);
}

// Float32 bit patterns of raw elements e and e + 1 (e even) of a float32 or
// BF16 array.
template <int ACT>
__device__ __forceinline__ uint2 load_pair(const char *base, int64_t e) {
    if (ACT == 0) return *(const uint2 *)(base + e * 4);
    const uint32_t w = *(const uint32_t *)(base + e * 2);
    return make_uint2(w << 16, w & 0xFFFF0000u);
}
__device__ __forceinline__ double dval(uint32_t bits) { return (double)__uint_as_float(bits); }

// Broadcast of lane r's double.
__device__ __forceinline__ double lane_bcast(double x, int r) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, r);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), r);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// The other half's double (lane l gets lane l ^ 32's value).
__device__ __forceinline__ double swap_halves(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)u, 32, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(u >> 32), 32, 64);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Encode pooled float32 pairs into a KV store row: no-RoPE pairs p = lane +
// 64 i (valid where 2p < Dn) and, where `rope_on`, RoPE pair `rp`.
__device__ __forceinline__ void store_kv_pairs(const KvView &s, int b, int64_t row, const float (&x0)[2],
                                               const float (&x1)[2], int ni, bool rope_on, int rp, float rx, float ry) {
    const int lane = lane_id();
    const int Dn = s.dim - ROPE_DIM;
    if (s.fmt == 0) {
        float *dst = (float *)(s.f32 + b * s.f32_bs + row * s.f32_rs);
        for (int i = 0; i < ni; ++i) {
            const int pr = lane + 64 * i;
            if (2 * pr < Dn) *(float2 *)&dst[2 * pr] = make_float2(x0[i], x1[i]);
        }
        if (rope_on) *(float2 *)&dst[Dn + 2 * rp] = make_float2(rx, ry);
        return;
    }
    // E4M3_BF16: dim 192, so the 128 no-RoPE dims are one group of pairs p = lane
    uint8_t c0, c1;
    const float sc = e4m3_group128(x0[0], x1[0], &c0, &c1);
    ((uint16_t *)(s.nope + b * s.nope_bs + row * s.nope_rs))[lane] = (uint16_t)(c0 | (c1 << 8));
    if (lane == 0) *(float *)(s.scale + b * s.scale_bs + row * s.scale_rs) = sc;
    if (rope_on)
        ((uint32_t *)(s.rope + b * s.rope_bs + row * s.rope_rs))[rp] =
            (uint32_t)bf16_encode(rx) | ((uint32_t)bf16_encode(ry) << 16);
}

// Encode pooled float32 pairs (dims 2p, 2p + 1, p = lane + 64 i) into the
// indexer store; every lane of the wave calls it. An MX block of 32 dims is
// one 16-lane row.
__device__ __forceinline__ void store_ik_pairs(const IkView &s, int b, int64_t entry, const float (&x0)[2],
                                               const float (&x1)[2], int ni, int dI) {
    const int lane = lane_id();
    for (int i = 0; i < ni; ++i) {
        const int pr = lane + 64 * i;
        const bool on = 2 * pr < dI;
        if (s.fmt == 0) {
            if (on) *(float2 *)&((float *)(s.f32 + b * s.f32_bs + entry * s.f32_rs))[2 * pr] = make_float2(x0[i], x1[i]);
            continue;
        }
        const bool bad = on && !(__builtin_isfinite(x0[i]) && __builtin_isfinite(x1[i]));
        float a = on ? amax_acc(amax_acc(0.0f, x0[i]), x1[i]) : 0.0f;
        a = __uint_as_float(row_max_u32(__float_as_uint(a)));
        const uint64_t row_bits = 0xFFFFull << (lane & 48);
        const bool nbad = (__ballot(bad) & row_bits) != 0;
        uint32_t code = 0;
        int E = 0;
        if (!nbad) {
            E = mx_exponent(a);
            code = e2m1_encode(__builtin_ldexpf(x0[i], -E)) | (e2m1_encode(__builtin_ldexpf(x1[i], -E)) << 4);
        }
        if (on) {
            ((uint8_t *)(s.e2m1 + b * s.e2m1_bs + entry * s.e2m1_rs))[pr] = (uint8_t)code;
            if ((lane & 15) == 0)
                ((uint8_t *)(s.e8m0 + b * s.e8m0_bs + entry * s.e8m0_rs))[pr >> 4] = nbad ? 0xFF : (uint8_t)(E + 127);
        }
    }
}

// Waves per (block, batch element, output) of the general kernel: wave w
// pools the w-th eighth of the block's tokens, and wave 0 adds the eight
// float64 partial sums in a fixed order (((w0 + w1) + (w2 + w3)) + ((w4 +
// w5) + (w6 + w7))) before the entry is rounded to float32 and encoded.
// Within a wave each value is a sum of four interleaved partial sums
// (independent FMA chains) over its tokens, added pairwise; its RoPE pair is
// pooled by both halves of the wave, each over half of the tokens (so K's
// float64 sin/cos run on every lane), the lower half's sum plus the upper's.
// Raw rows are read as pairs of elements, TB tokens' worth of loads at a time.
constexpr int CW = 8, TB = 8;

// Four interleaved partial sums: token s (counted from the first token of
// the run) goes to partial s % 4 while whole groups of four remain, to
// partial 0 after; the total is (a0 + a1) + (a2 + a3).
__device__ __forceinline__ double sum4(const double (&a)[4]) { return (a[0] + a[1]) + (a[2] + a[3]); }

// One workgroup per (block, batch element, output written); the outputs of a
// block are adjacent in blockIdx.x (x = n_out j + output: the K entry, the V
// entry, the indexer key, as far as they are written), so the costlier K
// workgroups spread over the device.
template <int ACT>
__global__ __launch_bounds__(64 * CW, 4) void compress_kernel(CompressPlan p) {
    __shared__ double alpha[MAX_M];
    __shared__ double part[CW][6][64];  // per wave: two pairs of pooled values per lane, then the RoPE pair
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const int n_out = (p.has_kv ? 2 : 0) + (p.has_ik ? 1 : 0);
    const int j = (int)(blockIdx.x / n_out);
    const int role = p.has_kv ? (int)(blockIdx.x % n_out) : 2;  // 0 K, 1 V, 2 indexer key
    const int b = blockIdx.y;
    const int m = p.m;
    const int64_t nblk = p.block_end ? 1 : p.t_new / m;
    const BlockGeo geo = block_geo(p, j, b, m);
    const int64_t tok0 = geo.tok0;                       // first raw row of the block
    const int64_t entry = geo.entry;
    // A ring store keeps only the last `ring` entries written by one call.
    const bool kv_keep = p.k.ring == 0 || (int64_t)j >= nblk - p.k.ring;
    if (!geo.ok || (role < 2 ? !(p.has_kv && kv_keep) : !p.has_ik)) return;  // uniform per workgroup

    // alpha_r = softmax_r(gate + pos_bias), float64, by wave 0
    if (wave == 0) {
        double zmax = -__builtin_inf();
        for (int r = lane; r < m; r += 64) {
            double z = (double)p.gate[(int64_t)b * p.t_new + tok0 + r] + (double)p.pos_bias[r];
            alpha[r] = z;
            zmax = z > zmax ? z : zmax;
        }
        zmax = wave_max(zmax);
        double zsum = 0.0;
        for (int r = lane; r < m; r += 64) {
            double e = exp(alpha[r] - zmax);
            alpha[r] = e;
            zsum += e;
        }
        zsum = wave_sum(zsum);
        for (int r = lane; r < m; r += 64) alpha[r] = alpha[r] / zsum;
    }
    __syncthreads();
    // this wave's tokens
    const int chunk = (m + CW - 1) / CW;
    const int r0 = wave * chunk < m ? wave * chunk : m;
    const int r1 = r0 + chunk < m ? r0 + chunk : m;
    const int n = r1 - r0, nfull = n & ~3;
    const int D = p.D, Dn = D - ROPE_DIM, dI = p.dI;
    const int width = role < 2 ? D : dI;
    const int n_el = role < 2 ? Dn : dI;  // elements pooled as pairs by every lane
    const int ni = n_el > 128 ? 2 : 1;
    const char *src = (const char *)(role == 0 ? p.raw_k : role == 1 ? p.raw_v : p.raw_ik);
    const int64_t rowbase = ((int64_t)b * p.t_new + tok0) * width;

    double a[2][2][4] = {};  // [pair i][element][partial]
    for (int rb = 0; rb < n; rb += TB) {
        uint2 x[TB][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i >= ni) break;  // uniform
            const int pr = lane + 64 * i;
            const int64_t off = 2 * pr < n_el ? 2 * pr : 0;
#pragma unroll
            for (int s = 0; s < TB; ++s) {
                const int r = rb + s < n ? r0 + rb + s : r0;
                x[s][i] = load_pair<ACT>(src, rowbase + (int64_t)r * width + off);
            }
        }
#pragma unroll
        for (int s = 0; s < TB; ++s) {
            if (rb + s >= n) break;  // uniform
            const double w = alpha[r0 + rb + s];
            const bool grouped = rb + s < nfull;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (i >= ni) break;
                if (grouped) {
                    a[i][0][s & 3] += w * dval(x[s][i].x);
                    a[i][1][s & 3] += w * dval(x[s][i].y);
                } else {
                    a[i][0][0] += w * dval(x[s][i].x);
                    a[i][1][0] += w * dval(x[s][i].y);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        part[wave][2 * i][lane] = sum4(a[i][0]);
        part[wave][2 * i + 1][lane] = sum4(a[i][1]);
    }
    if (role < 2) {
        // RoPE pair rp: the lower half pools tokens r0 .. r0 + nl - 1, the upper
        // half the rest; K is rotated at each token's position
        const bool up = lane >= 32;
        const int rp = lane & 31;
        const double f = p.inv_freq[rp];
        const int nl = (n + 1) / 2;
        const int ra = up ? r0 + nl : r0, nh = up ? n - nl : nl, nhf = nh & ~3;
        double ax[4] = {0.0, 0.0, 0.0, 0.0}, ay[4] = {0.0, 0.0, 0.0, 0.0};
        for (int rb = 0; rb < nl; rb += TB) {
            uint2 x[TB];
#pragma unroll
            for (int s = 0; s < TB; ++s) {
                const int r = rb + s < nh ? ra + rb + s : r0;
                x[s] = load_pair<ACT>(src, rowbase + (int64_t)r * width + Dn + 2 * rp);
            }
#pragma unroll
            for (int s = 0; s < TB; ++s) {
                if (rb + s >= nl) break;  // uniform; the upper half's extra slot is skipped below
                if (rb + s >= nh) continue;
                const int r = ra + rb + s;
                double xx = dval(x[s].x), yy = dval(x[s].y);
                if (role == 0) {
                    double sn, cs, xr, yr;
                    rope_sincos((double)(geo.first + r) * f, &sn, &cs);
                    rope_rotate(xx, yy, sn, cs, &xr, &yr);
                    xx = xr;
                    yy = yr;
                }
                const double w = alpha[r];
                if (rb + s < nhf) {
                    ax[s & 3] += w * xx;
                    ay[s & 3] += w * yy;
                } else {
                    ax[0] += w * xx;
                    ay[0] += w * yy;
                }
            }
        }
        const double hx = sum4(ax), hy = sum4(ay);
        const double ox = swap_halves(hx), oy = swap_halves(hy);
        if (!up) {
            part[wave][4][lane] = hx + ox;
            part[wave][5][lane] = hy + oy;
        }
    }
    __syncthreads();
    if (wave != 0) return;
    auto total = [&](int k) {
        return ((part[0][k][lane] + part[1][k][lane]) + (part[2][k][lane] + part[3][k][lane])) +
               ((part[4][k][lane] + part[5][k][lane]) + (part[6][k][lane] + part[7][k][lane]));
    };
    float x0[2], x1[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        x0[i] = (float)total(2 * i);
        x1[i] = (float)total(2 * i + 1);
    }
    if (role == 2) {
        store_ik_pairs(p.ik, b, entry, x0, x1, ni, dI);
        return;
    }
    float rx = 0.0f, ry = 0.0f;
    if (lane < ROPE_PAIRS) {
        rx = (float)total(4);
        ry = (float)total(5);
    }
    const KvView &dst = role == 0 ? p.k : p.v;
    store_kv_pairs(dst, b, kv_row(dst, entry), x0, x1, ni, lane < ROPE_PAIRS, lane, rx, ry);
}


// Blocks of at most SMALL_M tokens (the per-token window append, the CSA
// block). One wave per block and output written (the K entry, the V entry,
// the indexer key), so the encodes run side by side; the first wave evaluates
// the gate softmax for all of them.
// Every global load is issued before any arithmetic, so one memory round trip
// precedes the encode. Lane l holds element pairs (2p, 2p + 1), p = l + 64 i,
// of each row: a raw row is read as 32-bit words (two BF16 values) or 64-bit
// ones (two float32 values), and the encoders take two dims per lane. The
// float64 arithmetic is the general kernel's (gate softmax, RoPE, weighted
// sums, one rounding to float32), the sums running over the block's tokens
// in order (for m = 1 the pooling is skipped: it is the identity).
constexpr int SMALL_M = 4;

template <int ACT, int M>
__global__ __launch_bounds__(192) void compress_small_kernel(CompressPlan p) {
    // one wave per output written: K, V (when given), then the indexer key
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int role = p.has_kv ? wave : 2;
    const int j = blockIdx.x, b = blockIdx.y;
    const BlockGeo geo = block_geo(p, j, b, M);
    const int64_t tok0 = geo.tok0;
    const int64_t entry = geo.entry;
    const bool do_kv = p.has_kv && (p.k.ring == 0 || (int64_t)j >= (int64_t)gridDim.x - p.k.ring);
    if (!geo.ok) return;  // uniform per workgroup
    // K and V of an entry outside a ring store's kept rows are not written;
    // such waves still reach the barrier below and leave after it
    const bool active = role < 2 ? do_kv : true;
    const int D = p.D, Dn = D - ROPE_DIM;
    const int dI = p.dI;
    const int width = role < 2 ? D : dI;
    const int n_el = role < 2 ? Dn : dI;       // elements encoded as pairs by every lane
    const int ni = n_el > 128 ? 2 : 1;         // pairs per lane (at most 256 elements)
    // RoPE pairs: lanes 0..31 take the block's tokens 0 .. H-1, lanes 32..63
    // tokens H .. M-1, of pair lane & 31 (K's rotation is the costly part)
    constexpr int H = (M + 1) / 2;
    const bool up = lane >= 32;
    const int rp = lane & 31;
    const int rlo = up ? H : 0, rn = up ? M - H : H;  // this lane's RoPE tokens
    const char *src = (const char *)(role == 0 ? p.raw_k : role == 1 ? p.raw_v : p.raw_ik);
    const double f = p.inv_freq[rp];
    // Every load is unconditional, so all of them are in flight together: an
    // element past the row reads the row's first pair; values are masked after.
    float gz[M], gb[M];
    uint2 xn[M][2], xr[H];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const int64_t t = (int64_t)b * p.t_new + tok0 + r;
        gz[r] = p.gate[t];
        gb[r] = p.pos_bias[r];
        const int64_t row = t * width;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pr = lane + 64 * i;
            xn[r][i] = load_pair<ACT>(src, (i < ni && 2 * pr < n_el) ? row + 2 * pr : row);
        }
    }
    if (role < 2) {
#pragma unroll
        for (int u = 0; u < H; ++u) {
            const int r = rlo + u < M ? rlo + u : M - 1;
            xr[u] = load_pair<ACT>(src, ((int64_t)b * p.t_new + tok0 + r) * width + Dn + 2 * rp);
        }
    }
    // no load is sunk into the branches that use it (the register fence also
    // pins the rotation frequency, a kernel-argument load, up here)
    double fx = f;
    asm volatile("" : "+v"(fx) :: "memory");

    // alpha_r = softmax_r(gate + pos_bias) in float64, by the first wave for
    // all: lane r evaluates token r's exponential and quotient, the wave reads
    // them back (the sum runs over r = 0 .. M-1 in order) and lanes 0..M-1
    // publish the weights in LDS.
    __shared__ double s_alpha[SMALL_M];
    double alpha[M];
    if constexpr (M == 1) {
        alpha[0] = 1.0;
    } else {
        if (wave == 0) {
            double z[M];
#pragma unroll
            for (int r = 0; r < M; ++r) z[r] = (double)gz[r] + (double)gb[r];
            double zmax = z[0];
#pragma unroll
            for (int r = 1; r < M; ++r) zmax = z[r] > zmax ? z[r] : zmax;
            double zl = z[0];
#pragma unroll
            for (int r = 1; r < M; ++r) zl = lane == r ? z[r] : zl;
            const double el = exp(zl - zmax);
            double e[M], zsum = 0.0;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                e[r] = lane_bcast(el, r);
                zsum += e[r];
            }
            double eo = e[0];
#pragma unroll
            for (int r = 1; r < M; ++r) eo = lane == r ? e[r] : eo;
            const double al = eo / zsum;
            if (lane < M) s_alpha[lane] = al;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < M; ++r) alpha[r] = s_alpha[r];
    }
    if (!active) return;

    float x0[2] = {0.f, 0.f}, x1[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        if (i >= ni) break;
        if constexpr (M == 1) {
            x0[i] = __uint_as_float(xn[0][i].x);
            x1[i] = __uint_as_float(xn[0][i].y);
        } else {
            double a0 = 0.0, a1 = 0.0;
#pragma unroll
            for (int r = 0; r < M; ++r) {
                a0 += alpha[r] * dval(xn[r][i].x);
                a1 += alpha[r] * dval(xn[r][i].y);
            }
            x0[i] = (float)a0;
            x1[i] = (float)a1;
        }
    }
    if (role == 2) {
        store_ik_pairs(p.ik, b, entry, x0, x1, ni, dI);
        return;
    }
    // RoPE pair: K rotated at each token's position, V as it is; the lower
    // half's partial sums go to the upper half, which adds its tokens after
    // them (the order of a sequential sum over the block)
    float rx = 0.f, ry = 0.f;
    bool rope_on;
    if constexpr (M == 1) {
        if (role == 0) {
            double sn, cs, xa, ya;
            rope_sincos((double)geo.first * fx, &sn, &cs);
            rope_rotate(dval(xr[0].x), dval(xr[0].y), sn, cs, &xa, &ya);
            rx = (float)xa;
            ry = (float)ya;
        } else {
            rx = __uint_as_float(xr[0].x);
            ry = __uint_as_float(xr[0].y);
        }
        rope_on = !up;
    } else {
        double ax = 0.0, ay = 0.0;
        double px[H], py[H];
#pragma unroll
        for (int u = 0; u < H; ++u) {
            double x = dval(xr[u].x), y = dval(xr[u].y);
            if (role == 0 && u < rn) {
                double sn, cs, xa, ya;
                rope_sincos((double)(geo.first + rlo + u) * fx, &sn, &cs);
                rope_rotate(x, y, sn, cs, &xa, &ya);
                x = xa;
                y = ya;
            }
            px[u] = x;
            py[u] = y;
        }
        // lower half: tokens 0 .. H-1 from zero
#pragma unroll
        for (int u = 0; u < H; ++u) {
            ax += alpha[u] * px[u];
            ay += alpha[u] * py[u];
        }
        const double sx = swap_halves(ax), sy = swap_halves(ay);
        if (up) {
            ax = sx;
            ay = sy;
#pragma unroll
            for (int u = 0; u < M - H; ++u) {
                ax += alpha[H + u] * px[u];
                ay += alpha[H + u] * py[u];
            }
        }
        rx = (float)ax;
        ry = (float)ay;
        rope_on = up;
    }
    const KvView &dst = role == 0 ? p.k : p.v;
    store_kv_pairs(dst, b, kv_row(dst, entry), x0, x1, ni, rope_on, rp, rx, ry);
}

// Window rows (m = 1, a chunk of raw tokens): the pooling is the identity, so
// a wave encodes two consecutive tokens: both tokens' no-RoPE pairs on every
// lane, token 2g's RoPE pair on lanes 0..31 and token 2g + 1's on lanes 32..63
// (each half rotates its own token). One wave per output (K, V, indexer key),
// two waves when no indexer key is written. Bitwise the rows that
// compress_small_kernel<ACT, 1> writes.
template <int ACT>
__global__ __launch_bounds__(192) void compress_rows_kernel(CompressPlan p) {
    const int lane = lane_id(), role = threadIdx.x >> 6;
    const int b = blockIdx.y;
    const int64_t t0 = 2 * (int64_t)blockIdx.x;              // first token of the pair
    const int nt = t0 + 1 < p.t_new ? 2 : 1;                  // tokens of this pair (uniform)
    const int orole = p.has_kv ? role : 2;                    // output of this wave
    if (orole < 2 ? !p.has_kv : (!p.has_ik || role > (p.has_kv ? 2 : 0))) return;  // uniform per wave
    const int D = p.D, Dn = D - ROPE_DIM;
    const int dI = p.dI;
    const int width = orole < 2 ? D : dI;
    const int n_el = orole < 2 ? Dn : dI;
    const int ni = n_el > 128 ? 2 : 1;
    const bool up = lane >= 32;
    const int rp = lane & 31;
    const char *src = (const char *)(orole == 0 ? p.raw_k : orole == 1 ? p.raw_v : p.raw_ik);
    const double f = p.inv_freq[rp];
    uint2 xn[2][2], xr;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        const int64_t row = ((int64_t)b * p.t_new + t0 + (g < nt ? g : 0)) * width;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pr = lane + 64 * i;
            xn[g][i] = load_pair<ACT>(src, (i < ni && 2 * pr < n_el) ? row + 2 * pr : row);
        }
    }
    if (orole < 2) {
        const int g = up && nt > 1 ? 1 : 0;
        xr = load_pair<ACT>(src, ((int64_t)b * p.t_new + t0 + g) * width + Dn + 2 * rp);
    }
    double fx = f;
    asm volatile("" : "+v"(fx) :: "memory");
    if (orole == 2) {
#pragma unroll
        for (int g = 0; g < 2; ++g) {
            if (g >= nt) break;
            float x0[2], x1[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                x0[i] = __uint_as_float(xn[g][i].x);
                x1[i] = __uint_as_float(xn[g][i].y);
            }
            store_ik_pairs(p.ik, b, p.pos0 + t0 + g, x0, x1, ni, dI);
        }
        return;
    }
    // this half's token: K rotated at its position, V as it is
    const int64_t pos = p.pos0 + t0 + (up ? 1 : 0);
    float rx, ry;
    if (orole == 0) {
        double sn, cs, xa, ya;
        rope_sincos((double)pos * fx, &sn, &cs);
        rope_rotate(dval(xr.x), dval(xr.y), sn, cs, &xa, &ya);
        rx = (float)xa;
        ry = (float)ya;
    } else {
        rx = __uint_as_float(xr.x);
        ry = __uint_as_float(xr.y);
    }
    const KvView &dst = orole == 0 ? p.k : p.v;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
        if (g >= nt) break;
        // a ring store keeps only the chunk's last `ring` rows
        const int64_t tok = t0 + g;
        if (p.k.ring > 0 && tok < (int64_t)p.t_new - p.k.ring) continue;  // uniform
        float x0[2], x1[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            x0[i] = __uint_as_float(xn[g][i].x);
            x1[i] = __uint_as_float(xn[g][i].y);
        }
        store_kv_pairs(dst, b, kv_row(dst, p.pos0 + tok), x0, x1, ni, g == 0 ? !up : up, rp, rx, ry);
    }
}

// ------------------------------------------------------------ variants ----
// The compressor variants of v4a_pool_variant: overlapping windows of 2m,
// RoPE applied after pooling, one gate per token and channel. One wave per
// (block, batch element, output written), with the general kernel's float64
// arithmetic and one rounding to float32 before encoding. Lane l takes the
// element pairs (2p, 2p + 1), p = l + 64 i, of each row; a RoPE pair is pooled
// by both halves of the wave, each over half of the window's tokens (the
// lower half's sum plus the upper's), so each token is rotated once.

constexpr int MAX_VAR_WINDOW = 1024;  // tokens one entry pools (2m for overlapping windows)

template <int ACT, int VAR>
__global__ __launch_bounds__(64) void compress_var_kernel(CompressPlan p) {
    __shared__ double alpha[MAX_VAR_WINDOW];
    const int lane = lane_id();
    const int j = blockIdx.x, b = blockIdx.y;
    const int role = p.has_kv ? (int)blockIdx.z : 2;  // 0 K, 1 V, 2 indexer key (z: the outputs written)
    const int m = p.m;
    const BlockGeo geo = block_geo(p, j, b, m);
    const bool kv_keep = p.k.ring == 0 || (int64_t)j >= (int64_t)gridDim.x - p.k.ring;
    if (!geo.ok || (role < 2 ? !(p.has_kv && kv_keep) : !p.has_ik)) return;  // uniform per workgroup
    constexpr bool overlap = VAR == V4A_POOL_OVERLAP, chan = VAR == V4A_POOL_CHANNEL_GATE;
    const int wm = overlap ? 2 * m : m;                          // tokens of the window
    const int64_t wpos0 = overlap ? geo.first - m : geo.first;   // position of window token 0
    const int r0 = wpos0 < 0 ? (int)-wpos0 : 0;                  // tokens before position 0 take no part
    // raw rows of batch element b: a linear chunk (positions from pos0, or from pos0 - m for
    // overlapping windows) or, in block mode, a ring of t_new rows indexed by position
    const int64_t rows_b = p.block_end ? p.t_new : p.t_new + (overlap ? m : 0);
    auto row = [&](int r) -> int64_t { return p.block_end ? (wpos0 + r) % p.t_new : (int64_t)j * m + r; };
    const int C = p.gate_c;

    if (!chan) {
        // alpha_r = softmax over the window of (gate + pos_bias[r]), float64
        double zmax = -__builtin_inf();
        for (int r = r0 + lane; r < wm; r += 64) {
            const double z = (double)p.gate[(int64_t)b * rows_b + row(r)] + (double)p.pos_bias[r];
            alpha[r] = z;
            zmax = z > zmax ? z : zmax;
        }
        zmax = wave_max(zmax);
        double zsum = 0.0;
        for (int r = r0 + lane; r < wm; r += 64) {
            const double e = exp(alpha[r] - zmax);
            alpha[r] = e;
            zsum += e;
        }
        zsum = wave_sum(zsum);
        for (int r = r0 + lane; r < wm; r += 64) alpha[r] = alpha[r] / zsum;
        __syncthreads();
    }
    // per-channel gates: channel c's softmax over the window, its maximum and
    // sum taken over the tokens in order, then each token's weight
    auto zc = [&](int r, int c) -> double {
        return (double)p.gate[((int64_t)b * rows_b + row(r)) * C + c] + (double)p.pos_bias[(int64_t)r * C + c];
    };
    struct Norm {
        double zmax, zsum;
    };
    auto norm = [&](int c) -> Norm {
        Norm n{-__builtin_inf(), 0.0};
        if (!chan) return n;
        for (int r = r0; r < wm; ++r) {
            const double z = zc(r, c);
            n.zmax = z > n.zmax ? z : n.zmax;
        }
        for (int r = r0; r < wm; ++r) n.zsum += exp(zc(r, c) - n.zmax);
        return n;
    };
    auto weight = [&](int r, int c, const Norm &n) -> double {
        return chan ? exp(zc(r, c) - n.zmax) / n.zsum : alpha[r];
    };

    const int D = p.D, Dn = D - ROPE_DIM, dI = p.dI;
    const int width = role < 2 ? D : dI;
    const int n_el = role < 2 ? Dn : dI;  // elements pooled as pairs by every lane
    const int ni = n_el > 128 ? 2 : 1;
    const char *src = (const char *)(role == 0 ? p.raw_k : role == 1 ? p.raw_v : p.raw_ik);
    const int cbase = role == 0 ? 0 : role == 1 ? D : (p.has_kv ? 2 * D : 0);  // gate column of dim 0
    auto elem = [&](int r, int64_t e) { return load_pair<ACT>(src, ((int64_t)b * rows_b + row(r)) * width + e); };

    // pairs: four interleaved partial sums over the window from r0, whole
    // groups of four, then the rest into partial 0
    float x0[2] = {0.f, 0.f}, x1[2] = {0.f, 0.f};
    for (int i = 0; i < ni; ++i) {
        const int pr = lane + 64 * i;
        const bool on = 2 * pr < n_el;
        const int64_t e = on ? 2 * pr : 0;
        const int c0 = cbase + (int)e, c1 = c0 + 1;
        const Norm n0 = norm(c0), n1 = norm(c1);
        double a0[4] = {0.0, 0.0, 0.0, 0.0}, a1[4] = {0.0, 0.0, 0.0, 0.0};
        int r = r0;
        for (; r + 4 <= wm; r += 4) {
            uint2 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = elem(r + u, e);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                a0[u] += weight(r + u, c0, n0) * dval(v[u].x);
                a1[u] += weight(r + u, c1, n1) * dval(v[u].y);
            }
        }
        for (; r < wm; ++r) {
            const uint2 v = elem(r, e);
            a0[0] += weight(r, c0, n0) * dval(v.x);
            a1[0] += weight(r, c1, n1) * dval(v.y);
        }
        x0[i] = (float)sum4(a0);
        x1[i] = (float)sum4(a1);
    }
    if (role == 2) {
        store_ik_pairs(p.ik, b, geo.entry, x0, x1, ni, dI);
        return;
    }
    // RoPE pair rp: the lower half pools the window's first tokens, the upper
    // half the rest; keys rotated at each token's position, or (RoPE after
    // pooling) the pooled key once at the block's last position
    const bool up = lane >= 32;
    const int rp = lane & 31;
    const double f = p.inv_freq[rp];
    const bool rot_each = role == 0 && VAR != V4A_POOL_ROPE_AFTER;
    const int n = wm - r0, nl = (n + 1) / 2;
    const int ra = up ? r0 + nl : r0, nh = up ? n - nl : nl;
    const int cx = cbase + Dn + 2 * rp, cy = cx + 1;
    const Norm nx = norm(cx), ny = norm(cy);
    double ax[4] = {0.0, 0.0, 0.0, 0.0}, ay[4] = {0.0, 0.0, 0.0, 0.0};
    auto rope_tok = [&](int r, double *x, double *y) {
        const uint2 v = elem(r, Dn + 2 * rp);
        *x = dval(v.x);
        *y = dval(v.y);
        if (rot_each) {
            double sn, cs, xr, yr;
            rope_sincos((double)(wpos0 + r) * f, &sn, &cs);
            rope_rotate(*x, *y, sn, cs, &xr, &yr);
            *x = xr;
            *y = yr;
        }
    };
    int s = 0;
    for (; s + 4 <= nh; s += 4) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            double x, y;
            rope_tok(ra + s + u, &x, &y);
            ax[u] += weight(ra + s + u, cx, nx) * x;
            ay[u] += weight(ra + s + u, cy, ny) * y;
        }
    }
    for (; s < nh; ++s) {
        double x, y;
        rope_tok(ra + s, &x, &y);
        ax[0] += weight(ra + s, cx, nx) * x;
        ay[0] += weight(ra + s, cy, ny) * y;
    }
    const double hx = sum4(ax), hy = sum4(ay);
    const double ox = swap_halves(hx), oy = swap_halves(hy);
    double px = hx + ox, py = hy + oy;  // used on the lower half: its sum plus the upper's
    if (role == 0 && VAR == V4A_POOL_ROPE_AFTER) {
        double sn, cs, xr, yr;
        rope_sincos((double)(geo.first + m - 1) * f, &sn, &cs);
        rope_rotate(px, py, sn, cs, &xr, &yr);
        px = xr;
        py = yr;
    }
    const KvView &dst = role == 0 ? p.k : p.v;
    store_kv_pairs(dst, b, kv_row(dst, geo.entry), x0, x1, ni, !up, rp, (float)px, (float)py);
}

template <int ACT>
static void launch_variant(const CompressPlan &p, dim3 g3, hipStream_t s) {
    switch (p.variant) {
        case V4A_POOL_OVERLAP: hipLaunchKernelGGL((compress_var_kernel<ACT, V4A_POOL_OVERLAP>), g3, dim3(64), 0, s, p); break;
        case V4A_POOL_ROPE_AFTER: hipLaunchKernelGGL((compress_var_kernel<ACT, V4A_POOL_ROPE_AFTER>), g3, dim3(64), 0, s, p); break;
        default: hipLaunchKernelGGL((compress_var_kernel<ACT, V4A_POOL_CHANNEL_GATE>), g3, dim3(64), 0, s, p); break;
    }
}

template <int ACT>
static void launch_small(const CompressPlan &p, dim3 grid, hipStream_t s) {
    if (p.m == 1 && !p.block_end) {  // a chunk of window rows: two tokens per wave
        const dim3 g2((unsigned)((p.t_new + 1) / 2), grid.y);
        const unsigned nt = (p.has_kv ? 128u : 0u) + (p.has_ik ? 64u : 0u);
        hipLaunchKernelGGL((compress_rows_kernel<ACT>), g2, dim3(nt), 0, s, p);
        return;
    }
    const dim3 blk((p.has_kv ? 128 : 0) + (p.has_ik ? 64 : 0));  // one wave per output written
    switch (p.m) {
        case 1: hipLaunchKernelGGL((compress_small_kernel<ACT, 1>), grid, blk, 0, s, p); break;
        case 2: hipLaunchKernelGGL((compress_small_kernel<ACT, 2>), grid, blk, 0, s, p); break;
        case 3: hipLaunchKernelGGL((compress_small_kernel<ACT, 3>), grid, blk, 0, s, p); break;
        default: hipLaunchKernelGGL((compress_small_kernel<ACT, 4>), grid, blk, 0, s, p); break;
    }
}

hipError_t launch_compress(const CompressPlan &p, hipStream_t s) {
    dim3 grid(p.block_end ? 1 : p.t_new / p.m, p.B);  // block mode: one block per batch element
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (p.variant != V4A_POOL_BLOCK) {
        const dim3 g3(grid.x, grid.y, (p.has_kv ? 2u : 0u) + (p.has_ik ? 1u : 0u));  // the outputs written
        if (p.act == 0) launch_variant<0>(p, g3, s);
        else launch_variant<1>(p, g3, s);
    } else if (p.m <= SMALL_M) {
        if (p.act == 0) launch_small<0>(p, grid, s);
        else launch_small<1>(p, grid, s);
    } else {
        const unsigned n_out = (p.has_kv ? 2u : 0u) + (p.has_ik ? 1u : 0u);
        const dim3 gx(grid.x * n_out, grid.y);  // the outputs of each block side by side
        if (p.act == 0) hipLaunchKernelGGL(compress_kernel<0>, gx, dim3(64 * CW), 0, s, p);
        else hipLaunchKernelGGL(compress_kernel<1>, gx, dim3(64 * CW), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace v4a
