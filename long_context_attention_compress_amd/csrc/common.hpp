// Device helpers shared by the v4attn kernels (gfx950, wave64).
//
// Number formats (the pages name FP8, BF16, FP4/MXFP4 for the caches and the
// indexer; the encodings are the OCP ones):
//  * E4M3: OCP OFP8 rev 1.0 E4M3; round to nearest even, finite overflow
//    saturates to +-448, NaN -> 0x7F.
//  * BF16: top half of a float32 after round to nearest even.
//  * E2M1 + E8M0: OCP MX v1.0; shared exponent floor(log2 amax) - 2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "v4attn_internal.hpp"

namespace v4a {

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---------------------------------------------------------- kernel args ----
// Fetch every 64-byte line of a kernel's argument block into the scalar cache
// in one batch (one wait): the fields are read lazily all through a kernel,
// and each first touch of a line would otherwise be a round trip of its own.
template <typename T>
__device__ __forceinline__ void touch_args(const T &p) {
    static_assert(sizeof(T) <= 16 * 64, "the argument block spans at most 16 lines");
    const uint32_t *kp = (const uint32_t *)&p;
    constexpr int NL = (int)((sizeof(T) + 63) / 64);
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = i < NL ? kp[16 * i] : 0u;
    asm volatile("" ::"s"(w[0]), "s"(w[1]), "s"(w[2]), "s"(w[3]), "s"(w[4]), "s"(w[5]), "s"(w[6]), "s"(w[7]),
                 "s"(w[8]), "s"(w[9]), "s"(w[10]), "s"(w[11]), "s"(w[12]), "s"(w[13]), "s"(w[14]), "s"(w[15]));
}

// ------------------------------------------------------------ reductions ----
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        T u = __shfl_xor(v, o, 64);
        v = (u > v) ? u : v;
    }
    return v;
}
template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
// Max over a 32-lane half of the wave (lanes 0..31 and 32..63 reduce separately).
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
        float u = __shfl_xor(v, o, 64);
        v = (u > v || __builtin_isnan(u)) ? u : v;
    }
    return v;
}
// NaN-propagating max of magnitudes.
__device__ __forceinline__ float amax_acc(float m, float x) {
    float a = __builtin_fabsf(x);
    return (a > m || __builtin_isnan(a)) ? a : m;
}
__device__ __forceinline__ float wave_amax(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        float u = __shfl_xor(v, o, 64);
        v = (u > v || __builtin_isnan(u)) ? u : v;
    }
    return v;
}

// Unsigned max over a 16-lane row, a 32-lane half and the wave, on the VALU:
// DPP row rotations, then the gfx950 lane-swap instructions across rows.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
    uint32_t y;
    y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);  // row_ror:8
    x = y > x ? y : x;
    y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x124, 0xF, 0xF, false);  // row_ror:4
    x = y > x ? y : x;
    y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x122, 0xF, 0xF, false);  // row_ror:2
    x = y > x ? y : x;
    y = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x121, 0xF, 0xF, false);  // row_ror:1
    return y > x ? y : x;
}
__device__ __forceinline__ uint32_t half_max_u32(uint32_t x) {
    x = row_max_u32(x);
    auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return a[0] > a[1] ? a[0] : a[1];
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
    x = half_max_u32(x);
    auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return c[0] > c[1] ? c[0] : c[1];
}
// Float max and sum over the wave on the VALU (DPP row rotations, then the
// lane swaps), with the result in every lane. Each step combines a lane's
// value with one that its partner combines in the other order, so every lane
// ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float row_rot(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
    float y;
    y = row_rot<0x128>(x); x = y > x ? y : x;  // row_ror:8
    y = row_rot<0x124>(x); x = y > x ? y : x;  // row_ror:4
    y = row_rot<0x122>(x); x = y > x ? y : x;  // row_ror:2
    y = row_rot<0x121>(x); x = y > x ? y : x;  // row_ror:1
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) > __uint_as_float(a[1]) ? __uint_as_float(a[0]) : __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) > __uint_as_float(c[1]) ? __uint_as_float(c[0]) : __uint_as_float(c[1]);
}
__device__ __forceinline__ float wave_sum_dpp(float x) {
    x += row_rot<0x128>(x);
    x += row_rot<0x124>(x);
    x += row_rot<0x122>(x);
    x += row_rot<0x121>(x);
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// Magnitude maxima (inputs are |x| or a NaN with the sign cleared; as bits
// they order like the magnitudes, a NaN above infinity, so a NaN propagates).
__device__ __forceinline__ float wave_amax_bits(float a) { return __uint_as_float(wave_max_u32(__float_as_uint(a))); }
__device__ __forceinline__ float half_amax_bits(float a) { return __uint_as_float(half_max_u32(__float_as_uint(a))); }

// ------------------------------------------------------------------ BF16 ----
__device__ __forceinline__ uint16_t bf16_encode(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_decode(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// ------------------------------------------------------------------ E4M3 ----
__device__ __forceinline__ uint8_t e4m3_encode(float x) {
    if (__builtin_isnan(x)) return 0x7F;
    uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
    float a = __builtin_fabsf(x);
    if (a >= 448.0f) return (uint8_t)(sign | 0x7Eu);
    if (a < 0.015625f) {                        // subnormal range: quantum 2^-9
        float n = __builtin_rintf(a * 512.0f);  // exact scaling, round half to even
        return (uint8_t)(sign | (uint32_t)n);   // n == 8 is the smallest normal
    }
    int e = (int)((__float_as_uint(a) >> 23) & 0xFFu) - 127;  // floor(log2 a), a normal
    float sc = __builtin_rintf(__builtin_ldexpf(a, 3 - e));   // 8 .. 16
    uint32_t code = (uint32_t)((e + 7) << 3) + ((uint32_t)sc - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
    return (uint8_t)(sign | code);
}
__device__ __forceinline__ float e4m3_decode(uint8_t c) {
    uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
    float v;
    if (e == 15u && m == 7u) v = __builtin_nanf("");
    else if (e == 0u) v = (float)m * 0.001953125f;  // m/8 * 2^-6
    else v = __builtin_ldexpf(1.0f + (float)m * 0.125f, (int)e - 7);
    return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------- E2M1/MX ----
__device__ __forceinline__ uint32_t e2m1_encode(float v) {
    uint32_t s = __builtin_signbit(v) ? 8u : 0u;
    float a = __builtin_fabsf(v);
    uint32_t code;
    if (a < 2.0f) {
        code = (uint32_t)__builtin_rintf(a * 2.0f);  // 0..4 (4 == 2.0)
    } else if (a < 4.0f) {
        code = (uint32_t)__builtin_rintf(a) + 2u;   // 4..6
    } else {
        float q = __builtin_rintf(a * 0.5f);         // 2..
        code = q >= 3.0f ? 7u : 6u;                  // 4.0 -> 6, 6.0 (and above) -> 7
    }
    return s | code;
}
// Shared exponent of an MX block from its amax (finite); returns E.
__device__ __forceinline__ int mx_exponent(float amax) {
    uint32_t ex = (__float_as_uint(amax) >> 23) & 0xFFu;
    if (ex == 0u) return -127;                       // zero or subnormal amax
    int e = (int)ex - 127 - 2;
    return e < -127 ? -127 : e;
}

// ------------------------------------------------------------- RoPE angle ----
// sin and cos of a float64 angle. RoPE angles reach 1e6 radians at a million
// positions, where the library routine takes its slow large-argument path.
// Here: Cody-Waite reduction by pi/2 with pi/2 split into three doubles (the
// first two carry 28 significant bits, so n*P1 and n*P2 are exact for
// |n| < 2^25), then Taylor polynomials on |r| <= pi/4 (terms to r^23, error
// below 1e-27). Angles beyond 2^25 * pi/2 fall back to the library routine.
__device__ __forceinline__ void rope_sincos(double x, double *sn, double *cs) {
    const double ax = __builtin_fabs(x);
    if (!(ax < 5.2e7)) {  // also catches NaN
        sincos(x, sn, cs);
        return;
    }
    const double P1 = 0x1.921fb54000000p+0, P2 = 0x1.10b4610000000p-30, P3 = 0x1.a62633145c06ep-58;
    const double n = __builtin_rint(x * 0x1.45f306dc9c883p-1);  // x * 2/pi
    const double r = ((x - n * P1) - n * P2) - n * P3;
    const double r2 = r * r;
    // sin r = r (1 - r^2/3! + r^4/5! - ...), cos r = 1 - r^2/2! + r^4/4! - ...
    double ps = -1.0 / 25852016738884976640000.0;  // -1/23!
    ps = __builtin_fma(ps, r2, 1.0 / 51090942171709440000.0);
    ps = __builtin_fma(ps, r2, -1.0 / 121645100408832000.0);
    ps = __builtin_fma(ps, r2, 1.0 / 355687428096000.0);
    ps = __builtin_fma(ps, r2, -1.0 / 1307674368000.0);
    ps = __builtin_fma(ps, r2, 1.0 / 6227020800.0);
    ps = __builtin_fma(ps, r2, -1.0 / 39916800.0);
    ps = __builtin_fma(ps, r2, 1.0 / 362880.0);
    ps = __builtin_fma(ps, r2, -1.0 / 5040.0);
    ps = __builtin_fma(ps, r2, 1.0 / 120.0);
    ps = __builtin_fma(ps, r2, -1.0 / 6.0);
    const double s = __builtin_fma(ps * r2, r, r);
    double pc = 1.0 / 1124000727777607680000.0;     // 1/22!
    pc = __builtin_fma(pc, r2, -1.0 / 2432902008176640000.0);
    pc = __builtin_fma(pc, r2, 1.0 / 6402373705728000.0);
    pc = __builtin_fma(pc, r2, -1.0 / 20922789888000.0);
    pc = __builtin_fma(pc, r2, 1.0 / 87178291200.0);
    pc = __builtin_fma(pc, r2, -1.0 / 479001600.0);
    pc = __builtin_fma(pc, r2, 1.0 / 3628800.0);
    pc = __builtin_fma(pc, r2, -1.0 / 40320.0);
    pc = __builtin_fma(pc, r2, 1.0 / 720.0);
    pc = __builtin_fma(pc, r2, -1.0 / 24.0);
    pc = __builtin_fma(pc, r2, 0.5);
    const double c = __builtin_fma(-pc, r2, 1.0);
    switch (((long long)n) & 3) {
        case 0: *sn = s; *cs = c; break;
        case 1: *sn = c; *cs = -s; break;
        case 2: *sn = -s; *cs = -c; break;
        default: *sn = -c; *cs = s; break;
    }
}

// One RoPE pair rotated by the angle with sine sn and cosine cs, in float64.
// Contraction is off, so every kernel that rotates a raw key row (the
// compressor and the attention kernels' fused window append) rounds the same
// products the same way and writes the same bits.
__device__ __forceinline__ void rope_rotate(double x, double y, double sn, double cs, double *xr, double *yr) {
#pragma clang fp contract(off)
    *xr = x * cs - y * sn;
    *yr = x * sn + y * cs;
}

// ---------------------------------------------------------- E4M3 KV rows ----
// E4M3 codes of one 128-dim no-RoPE group that a wave holds as two values per
// lane (any two dims: each code depends only on its value and the group's
// scale), under the group's float32 scale amax / 448 (1 for an all-zero
// group; a NaN in the group makes the scale, and so every code, NaN).
// Returns the scale.
__device__ __forceinline__ float e4m3_group128(float x0, float x1, uint8_t *c0, uint8_t *c1) {
    float a = amax_acc(0.0f, x0);
    a = amax_acc(a, x1);
    a = wave_amax_bits(a);
    float sc = a > 0.0f ? __fdiv_rn(a, 448.0f) : 1.0f;
    if (__builtin_isnan(a)) sc = a;
    *c0 = e4m3_encode(__fdiv_rn(x0, sc));
    *c1 = e4m3_encode(__fdiv_rn(x1, sc));
    return sc;
}

// --------------------------------------------------- order-preserving key ----
// Larger float -> larger key; -0 == +0; NaN -> 0 (below every number).
__device__ __forceinline__ uint32_t score_key(float s) {
    if (__builtin_isnan(s)) return 0u;
    uint32_t u = __float_as_uint(s + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_score(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

}  // namespace v4a
