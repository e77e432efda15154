// csa_compress: softmax-gated pooling of m raw tokens into one cache entry.
//
// [chaosnode.de, "DeepSeek-V4: 1 Million Token Context endlich nutzbar",
// section "Hybrid Attention: CSA und HCA"]: CSA compresses KV entries 4x along
// the sequence by softmax-gated pooling with a learned positional bias; HCA
// compresses 128x. [golem.de, "... Bei Deepseek V4 haben kleine Änderungen
// große Wirkung", section "Komprimierte Erinnerung für längere Kontexte"]: the
// last 64 values carry RoPE and stay BF16, the rest is FP8.
//
// Four waves per (entry, batch element, output) for long blocks (a quarter
// of the tokens each), three waves (one per output) in one workgroup for
// blocks of up to four tokens. The gate weights, the RoPE rotation and the
// weighted sum are evaluated in float64 and the entry is rounded to float32
// before it is encoded, so every encoding decision (FP8 scale and codes, BF16
// rounding, MX exponent and E2M1 codes) is taken on a float32 value.
// Compression is a small share of decode time (one block per m tokens), so the
// kernels favour exactness over speed.

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

// sum_r alpha[r] * x(r) over r0 <= r < r1 in float64, as four interleaved
// partial sums (independent FMA chains) added pairwise at the end.
template <class F>
__device__ __forceinline__ double pooled(const double *alpha, int r0, int r1, F x) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int r = r0;
    for (; r + 4 <= r1; r += 4) {
        a0 += alpha[r] * x(r);
        a1 += alpha[r + 1] * x(r + 1);
        a2 += alpha[r + 2] * x(r + 2);
        a3 += alpha[r + 3] * x(r + 3);
    }
    for (; r < r1; ++r) a0 += alpha[r] * x(r);
    return (a0 + a1) + (a2 + a3);
}

// Waves per (block, batch element, output) of the general kernel: wave w
// pools the w-th quarter of the block's tokens, and wave 0 adds the four
// float64 partial sums in a fixed order ((w0 + w1) + (w2 + w3)) before the
// entry is rounded to float32 and encoded. (With one wave per output the
// m = 128 blocks of a chunked prefill ran as 128 waves on the whole device,
// each through 128 tokens and their float64 sin/cos: 120 us per call.)
constexpr int CW = 4;

// One workgroup per (block, batch element, output): blockIdx.z = 0 the K
// entry, 1 the V entry, 2 the indexer key.
template <int ACT>
__global__ __launch_bounds__(64 * CW) void compress_kernel(CompressPlan p) {
    __shared__ double alpha[MAX_M];
    __shared__ double part[CW][6][64];  // per wave: up to four pooled dims per lane, then the RoPE pair
    const int lane = lane_id();
    const int wave = (int)(threadIdx.x >> 6);
    const int j = blockIdx.x;  // block within the chunk
    const int b = blockIdx.y;
    const int role = blockIdx.z;
    const int m = p.m;
    const BlockGeo geo = block_geo(p, j, b, m);
    const int64_t tok0 = geo.tok0;                       // first raw row of the block
    const int64_t entry = geo.entry;
    // A ring store keeps only the last `ring` entries written by one call.
    const bool kv_keep = p.k.ring == 0 || (int64_t)j >= (int64_t)gridDim.x - p.k.ring;
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

    if (role < 2) {
        // values (never rotated) and keys (rotated at each token's position)
        const int D = p.D, Dn = D - ROPE_DIM, nit = Dn / 64;
        const int64_t rowbase = ((int64_t)b * p.t_new + tok0) * D;
        const void *src = role == 0 ? p.raw_k : p.raw_v;
        for (int i = 0; i < nit; ++i)
            part[wave][i][lane] = pooled(alpha, r0, r1, [&](int r) {
                return load_act<ACT>(src, rowbase + (int64_t)r * D + lane + 64 * i);
            });
        if (lane < ROPE_PAIRS) {
            const double f = p.inv_freq[lane];
            auto pair = [&](int r, double *x, double *y) {
                *x = load_act<ACT>(src, rowbase + (int64_t)r * D + Dn + 2 * lane);
                *y = load_act<ACT>(src, rowbase + (int64_t)r * D + Dn + 2 * lane + 1);
                if (role == 0) {
                    double sn, cs, xr, yr;
                    rope_sincos((double)(geo.first + r) * f, &sn, &cs);
                    rope_rotate(*x, *y, sn, cs, &xr, &yr);
                    *x = xr;
                    *y = yr;
                }
            };
            double ax[4] = {0.0, 0.0, 0.0, 0.0}, ay[4] = {0.0, 0.0, 0.0, 0.0};
            int r = r0;
            for (; r + 4 <= r1; r += 4)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    double x, y;
                    pair(r + u, &x, &y);
                    ax[u] += alpha[r + u] * x;
                    ay[u] += alpha[r + u] * y;
                }
            for (; r < r1; ++r) {
                double x, y;
                pair(r, &x, &y);
                ax[0] += alpha[r] * x;
                ay[0] += alpha[r] * y;
            }
            part[wave][4][lane] = (ax[0] + ax[1]) + (ax[2] + ax[3]);
            part[wave][5][lane] = (ay[0] + ay[1]) + (ay[2] + ay[3]);
        }
        __syncthreads();
        if (wave != 0) return;
        auto total = [&](int k) {
            return (part[0][k][lane] + part[1][k][lane]) + (part[2][k][lane] + part[3][k][lane]);
        };
        float nope[4];
        for (int i = 0; i < nit; ++i) nope[i] = (float)total(i);
        float rx = 0.0f, ry = 0.0f;
        if (lane < ROPE_PAIRS) {
            rx = (float)total(4);
            ry = (float)total(5);
        }
        const KvView &dst = role == 0 ? p.k : p.v;
        store_kv_row(dst, b, kv_row(dst, entry), nope, nit, rx, ry);
    } else {
        const int dI = p.dI, nit = dI / 64 + (dI % 64 ? 1 : 0);
        const int64_t rowbase = ((int64_t)b * p.t_new + tok0) * dI;
        for (int i = 0; i < nit; ++i) {
            const int d = lane + 64 * i;
            part[wave][i][lane] = d < dI ? pooled(alpha, r0, r1, [&](int r) {
                return load_act<ACT>(p.raw_ik, rowbase + (int64_t)r * dI + d);
            }) : 0.0;
        }
        __syncthreads();
        if (wave != 0) return;
        for (int i = 0; i < nit; ++i) {
            const int d = lane + 64 * i;
            const double acc = (part[0][i][lane] + part[1][i][lane]) + (part[2][i][lane] + part[3][i][lane]);
            store_ik_value(p.ik, b, entry, d, d < dI, (float)acc);
        }
    }
}

// Blocks of at most SMALL_M tokens (the per-token window append, the CSA
// block): every global load is issued before any arithmetic, so one memory
// round trip precedes the encode, and each lane evaluates the gate softmax
// itself. Same float64 arithmetic as the general kernel (for m = 1 the
// pooling is skipped: it is the identity).
constexpr int SMALL_M = 4;

// Raw bits of one activation (float32 or BF16) and its float32 value.
template <int ACT>
__device__ __forceinline__ uint32_t load_bits(const char *base, int64_t i) {
    if (ACT == 0) return ((const uint32_t *)base)[i];
    return ((const uint16_t *)base)[i];
}
template <int ACT>
__device__ __forceinline__ float bits_val(uint32_t x) {
    return ACT == 0 ? __uint_as_float(x) : __uint_as_float(x << 16);
}

// Three waves per block of tokens, one per output: wave 0 the K entry, wave
// 1 the V entry, wave 2 the indexer key (each evaluates the gate softmax
// itself), so the three encodes run side by side.
template <int ACT, int M>
__global__ __launch_bounds__(192) void compress_small_kernel(CompressPlan p) {
    const int lane = lane_id(), role = threadIdx.x >> 6;
    const int j = blockIdx.x, b = blockIdx.y;
    const BlockGeo geo = block_geo(p, j, b, M);
    const int64_t tok0 = geo.tok0;
    const int64_t entry = geo.entry;
    const bool do_kv = p.has_kv && (p.k.ring == 0 || (int64_t)j >= (int64_t)gridDim.x - p.k.ring);
    if (!geo.ok || (role < 2 ? !do_kv : !p.has_ik)) return;  // uniform per wave
    const int D = p.D, Dn = D - ROPE_DIM, nit = Dn / 64;
    const int dI = p.dI;
    const int width = role < 2 ? D : dI;
    const bool rl = lane < ROPE_PAIRS;
    // Every load is unconditional, so all of them are in flight together: an
    // element past the row reads the row's first; the values are masked after
    // the loads.
    const char *src = (const char *)(role == 0 ? p.raw_k : role == 1 ? p.raw_v : p.raw_ik);
    double f = p.inv_freq[rl ? lane : 0];
    float gz[M], gb[M];
    uint32_t xn[M][4], xa[M], xb[M];
#pragma unroll
    for (int r = 0; r < M; ++r) {
        const int64_t t = (int64_t)b * p.t_new + tok0 + r;
        gz[r] = p.gate[t];
        gb[r] = p.pos_bias[r];
        const int64_t row = t * width;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool on = role < 2 ? i < nit : lane + 64 * i < dI;
            xn[r][i] = load_bits<ACT>(src, on ? row + lane + 64 * i : row);
        }
        const int64_t xr = (role < 2 && rl) ? row + Dn + 2 * lane : row;
        xa[r] = load_bits<ACT>(src, xr);
        xb[r] = load_bits<ACT>(src, xr + ((role < 2 && rl) ? 1 : 0));
    }
    // no load is sunk into the branches that use it (the register fence also
    // pins the rotation frequency, a kernel-argument load, up here)
    asm volatile("" : "+v"(f) :: "memory");
    double z[M];
#pragma unroll
    for (int r = 0; r < M; ++r) z[r] = (double)gz[r] + (double)gb[r];
    // alpha_r = softmax_r(gate + pos_bias), float64
    double zmax = z[0];
#pragma unroll
    for (int r = 1; r < M; ++r) zmax = z[r] > zmax ? z[r] : zmax;
    double e[M], zsum = 0.0;
#pragma unroll
    for (int r = 0; r < M; ++r) {
        e[r] = exp(z[r] - zmax);
        zsum += e[r];
    }
    double alpha[M];
#pragma unroll
    for (int r = 0; r < M; ++r) alpha[r] = e[r] / zsum;

    if (role < 2) {
        // K (rotated at each token's position) or V
        float nx[4];
        float rx = 0.f, ry = 0.f;
        if constexpr (M == 1) {
            // one token: the pooling is the identity (alpha = 1 for any finite
            // gate) and the gate is not used. The attention kernels' fused
            // window append computes this same row with the same operations.
#pragma unroll
            for (int i = 0; i < 4; ++i) nx[i] = bits_val<ACT>(xn[0][i]);
            if (rl) {
                if (role == 0) {
                    double sn, cs, xr, yr;
                    rope_sincos((double)geo.first * f, &sn, &cs);
                    rope_rotate((double)bits_val<ACT>(xa[0]), (double)bits_val<ACT>(xb[0]), sn, cs, &xr, &yr);
                    rx = (float)xr;
                    ry = (float)yr;
                } else {
                    rx = bits_val<ACT>(xa[0]);
                    ry = bits_val<ACT>(xb[0]);
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                double a = 0.0;
#pragma unroll
                for (int r = 0; r < M; ++r) a += alpha[r] * (double)bits_val<ACT>(xn[r][i]);
                nx[i] = (float)a;
            }
            if (rl) {
                double ax = 0.0, ay = 0.0;
#pragma unroll
                for (int r = 0; r < M; ++r) {
                    double x = (double)bits_val<ACT>(xa[r]), y = (double)bits_val<ACT>(xb[r]);
                    if (role == 0) {
                        double sn, cs, xr, yr;
                        rope_sincos((double)(geo.first + r) * f, &sn, &cs);
                        rope_rotate(x, y, sn, cs, &xr, &yr);
                        x = xr;
                        y = yr;
                    }
                    ax += alpha[r] * x;
                    ay += alpha[r] * y;
                }
                rx = (float)ax;
                ry = (float)ay;
            }
        }
        const KvView &dst = role == 0 ? p.k : p.v;
        store_kv_row(dst, b, kv_row(dst, entry), nx, nit, rx, ry);
    } else {
        const int nit_i = (dI + 63) / 64;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i >= nit_i) break;
            const int d = lane + 64 * i;
            float x;
            if constexpr (M == 1) {
                x = bits_val<ACT>(d < dI ? xn[0][i] : 0u);
            } else {
                double acc = 0.0;
#pragma unroll
                for (int r = 0; r < M; ++r) acc += alpha[r] * (double)bits_val<ACT>(d < dI ? xn[r][i] : 0u);
                x = (float)acc;
            }
            store_ik_value(p.ik, b, entry, d, d < dI, x);
        }
    }
}

// ------------------------------------------------------------ variants ----
// The compressor variants of v4a_pool_variant: overlapping windows of 2m,
// RoPE applied after pooling, one gate per token and channel. One wave per
// (block, batch element, output), as compress_kernel, with the same float64
// arithmetic and float32 rounding before encoding.

constexpr int MAX_VAR_WINDOW = 1024;  // tokens one entry pools (2m for overlapping windows)

// sum over window tokens r0 .. n-1 of w(r) * x(r) in float64, four partial sums
template <class Wf, class Xf>
__device__ __forceinline__ double pool_window(int r0, int n, Wf w, Xf x) {
    double a0 = 0.0, a1 = 0.0, a2 = 0.0, a3 = 0.0;
    int r = r0;
    for (; r + 4 <= n; r += 4) {
        a0 += w(r) * x(r);
        a1 += w(r + 1) * x(r + 1);
        a2 += w(r + 2) * x(r + 2);
        a3 += w(r + 3) * x(r + 3);
    }
    for (; r < n; ++r) a0 += w(r) * x(r);
    return (a0 + a1) + (a2 + a3);
}

template <int ACT, int VAR>
__global__ __launch_bounds__(64) void compress_var_kernel(CompressPlan p) {
    __shared__ double alpha[MAX_VAR_WINDOW];
    const int lane = lane_id();
    const int j = blockIdx.x, b = blockIdx.y, role = blockIdx.z;
    const int m = p.m;
    const BlockGeo geo = block_geo(p, j, b, m);
    const bool kv_keep = p.k.ring == 0 || (int64_t)j >= (int64_t)gridDim.x - p.k.ring;
    if (!geo.ok || (role < 2 ? !(p.has_kv && kv_keep) : !p.has_ik)) return;  // uniform per workgroup
    const bool overlap = VAR == V4A_POOL_OVERLAP;
    const int wm = overlap ? 2 * m : m;                          // tokens of the window
    const int64_t wpos0 = overlap ? geo.first - m : geo.first;   // position of window token 0
    const int r0 = wpos0 < 0 ? (int)-wpos0 : 0;                  // tokens before position 0 take no part
    // raw rows of batch element b: a linear chunk (positions from pos0, or from pos0 - m for
    // overlapping windows) or, in block mode, a ring of t_new rows indexed by position
    const int64_t rows_b = p.block_end ? p.t_new : p.t_new + (overlap ? m : 0);
    auto row = [&](int r) -> int64_t { return p.block_end ? (wpos0 + r) % p.t_new : (int64_t)j * m + r; };
    const int C = p.gate_c;

    if (VAR != V4A_POOL_CHANNEL_GATE) {
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
    // pooled value of channel c (gate column c) of the rows given by x(r)
    auto pooled_ch = [&](int c, auto x) -> double {
        if (VAR != V4A_POOL_CHANNEL_GATE) return pool_window(r0, wm, [&](int r) { return alpha[r]; }, x);
        double zmax = -__builtin_inf();
        for (int r = r0; r < wm; ++r) {
            const double z = (double)p.gate[((int64_t)b * rows_b + row(r)) * C + c] + (double)p.pos_bias[(int64_t)r * C + c];
            zmax = z > zmax ? z : zmax;
        }
        double zsum = 0.0;
        for (int r = r0; r < wm; ++r)
            zsum += exp((double)p.gate[((int64_t)b * rows_b + row(r)) * C + c] + (double)p.pos_bias[(int64_t)r * C + c] - zmax);
        return pool_window(r0, wm, [&](int r) {
            return exp((double)p.gate[((int64_t)b * rows_b + row(r)) * C + c] + (double)p.pos_bias[(int64_t)r * C + c] - zmax) / zsum;
        }, x);
    };

    if (role < 2) {
        const int D = p.D, Dn = D - ROPE_DIM, nit = Dn / 64;
        const void *src = role == 0 ? p.raw_k : p.raw_v;
        const int cbase = role == 0 ? 0 : D;  // gate column of dim 0 of this output
        float nope[4];
        for (int i = 0; i < nit; ++i) {
            const int d = lane + 64 * i;
            nope[i] = (float)pooled_ch(cbase + d, [&](int r) { return load_act<ACT>(src, ((int64_t)b * rows_b + row(r)) * D + d); });
        }
        float rx = 0.0f, ry = 0.0f;
        if (lane < ROPE_PAIRS) {
            const double f = p.inv_freq[lane];
            const bool rot_each = role == 0 && VAR != V4A_POOL_ROPE_AFTER;  // keys rotated at each token's position
            auto pair = [&](int r, double *x, double *y) {
                const int64_t base = ((int64_t)b * rows_b + row(r)) * D + Dn + 2 * lane;
                *x = load_act<ACT>(src, base);
                *y = load_act<ACT>(src, base + 1);
                if (rot_each) {
                    double sn, cs, xr, yr;
                    rope_sincos((double)(wpos0 + r) * f, &sn, &cs);
                    rope_rotate(*x, *y, sn, cs, &xr, &yr);
                    *x = xr;
                    *y = yr;
                }
            };
            double px = pooled_ch(cbase + Dn + 2 * lane, [&](int r) { double x, y; pair(r, &x, &y); return x; });
            double py = pooled_ch(cbase + Dn + 2 * lane + 1, [&](int r) { double x, y; pair(r, &x, &y); return y; });
            if (role == 0 && VAR == V4A_POOL_ROPE_AFTER) {
                // the pooled key rotated once, at the block's last position
                double sn, cs, xr, yr;
                rope_sincos((double)(geo.first + m - 1) * f, &sn, &cs);
                rope_rotate(px, py, sn, cs, &xr, &yr);
                px = xr;
                py = yr;
            }
            rx = (float)px;
            ry = (float)py;
        }
        const KvView &dst = role == 0 ? p.k : p.v;
        store_kv_row(dst, b, kv_row(dst, geo.entry), nope, nit, rx, ry);
    } else {
        const int dI = p.dI, nit = dI / 64 + (dI % 64 ? 1 : 0);
        const int cbase = p.has_kv ? 2 * p.D : 0;
        for (int i = 0; i < nit; ++i) {
            const int d = lane + 64 * i;
            const bool on = d < dI;
            const double acc = on ? pooled_ch(cbase + d, [&](int r) {
                return load_act<ACT>(p.raw_ik, ((int64_t)b * rows_b + row(r)) * dI + d);
            }) : 0.0;
            store_ik_value(p.ik, b, geo.entry, d, on, (float)acc);
        }
    }
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
    switch (p.m) {
        case 1: hipLaunchKernelGGL((compress_small_kernel<ACT, 1>), grid, dim3(192), 0, s, p); break;
        case 2: hipLaunchKernelGGL((compress_small_kernel<ACT, 2>), grid, dim3(192), 0, s, p); break;
        case 3: hipLaunchKernelGGL((compress_small_kernel<ACT, 3>), grid, dim3(192), 0, s, p); break;
        default: hipLaunchKernelGGL((compress_small_kernel<ACT, 4>), grid, dim3(192), 0, s, p); break;
    }
}

hipError_t launch_compress(const CompressPlan &p, hipStream_t s) {
    dim3 grid(p.block_end ? 1 : p.t_new / p.m, p.B);  // block mode: one block per batch element
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (p.variant != V4A_POOL_BLOCK) {
        const dim3 g3(grid.x, grid.y, 3);  // K, V, indexer key
        if (p.act == 0) launch_variant<0>(p, g3, s);
        else launch_variant<1>(p, g3, s);
    } else if (p.m <= SMALL_M) {
        if (p.act == 0) launch_small<0>(p, grid, s);
        else launch_small<1>(p, grid, s);
    } else {
        const dim3 g3(grid.x, grid.y, 3);  // K, V, indexer key
        if (p.act == 0) hipLaunchKernelGGL(compress_kernel<0>, g3, dim3(64 * CW), 0, s, p);
        else hipLaunchKernelGGL(compress_kernel<1>, g3, dim3(64 * CW), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace v4a
