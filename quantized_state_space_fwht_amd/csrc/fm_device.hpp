// Device-side fixed-point helpers and the nonlinear approximation unit (NAU).
//
// Power-of-two fixed point ("What carries the argument" on the FastMamba review
// page: scales 2^p turn rescaling into shifts) and the shared exponential unit:
// an 8-segment first-order (chord) approximation of 2^v, e^x = 2^(x log2 e), and
// SoftPlus(x) = x + SoftPlus(-x) (Eq. (5), Section III-B.2; verdict record
// citations [15] and [16]).  SiLU reuses the unit through SiLU(x) = x + SiLU(-x).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

constexpr int kPMin = -24;
constexpr int kPMax = 24;
constexpr int64_t kClampLim = (int64_t)1 << 62;

__device__ __forceinline__ int32_t sat32(int64_t v) {
    return v > INT32_MAX ? INT32_MAX : (v < INT32_MIN ? INT32_MIN : (int32_t)v);
}

__device__ __forceinline__ int8_t sat8(int64_t v) {
    return (int8_t)(v > 127 ? 127 : (v < -127 ? -127 : v));
}

// floor(v * 2^-s + 1/2) for |v| < 2^62.  s < 0 is an exact left shift whose
// result is clamped to +-2^62 (every caller saturates to int32 afterwards).
__device__ __forceinline__ int64_t rshr(int64_t v, int s) {
    if (s > 0) {
        if (s >= 63) return 0;
        return (v + ((int64_t)1 << (s - 1))) >> s;
    }
    if (s == 0) return v;
    int k = -s;
    if (k >= 62) return v == 0 ? 0 : (v > 0 ? kClampLim : -kClampLim);
    int64_t lim = kClampLim >> k;
    v = v > lim ? lim : (v < -lim ? -lim : v);
    return v << k;
}

// rint()ed float32 -> int32 with saturation.
__device__ __forceinline__ int32_t f2i_sat(float f) {
    if (f >= 2147483648.0f) return INT32_MAX;
    if (f < -2147483648.0f) return INT32_MIN;
    return (int32_t)f;
}

// Largest p in [kPMin, kPMax] with a * 2^p <= 127 (a >= 0 float32); 0 for a == 0.
__device__ __forceinline__ int pot_from_f32(float a) {
    if (!(a > 0.0f)) return 0;
    double ad = (double)a;
    for (int p = kPMax; p > kPMin; --p)
        if (ad * __builtin_ldexp(1.0, p) <= 127.0) return p;
    return kPMin;
}

// Largest p in [kPMin, kPMax] with (m / 2^16) * 2^p <= 127 for a Q.16 maximum m >= 0.
__device__ __forceinline__ int pot_from_q16(int64_t m) {
    if (m <= 0) return 0;
    const int64_t lim = (int64_t)127 << 16;
    for (int p = kPMax; p > kPMin; --p) {
        bool ok = p >= 0 ? ((m << p) <= lim) : (m <= (lim << (-p)));
        if (ok) return p;
    }
    return kPMin;
}

// ---------------------------------------------------------------- NAU
// Chord endpoints Y_i = rint(2^(i/8) * 2^30), i = 0..8.
__device__ __forceinline__ int64_t exp2_knot(uint32_t i) {
    switch (i) {
        case 0: return 1073741824LL;
        case 1: return 1170923762LL;
        case 2: return 1276901417LL;
        case 3: return 1392470869LL;
        case 4: return 1518500250LL;
        case 5: return 1655936265LL;
        case 6: return 1805811301LL;
        case 7: return 1969251188LL;
        default: return 2147483648LL;
    }
}
constexpr int64_t kLog2eQ30 = 1549082005LL;  // rint(log2(e) * 2^30)

// 2^(v/2^16) in Q.16 for v <= 0 (result in [0, 2^16]).
__device__ __forceinline__ int32_t nau_exp2(int64_t v) {
    if (v < -((int64_t)32 << 16)) return 0;
    int64_t n = v >> 16;                       // floor of the integer part
    uint32_t f = (uint32_t)(v - (n << 16));    // [0, 2^16)
    uint32_t seg = f >> 13;                    // chord 0..7
    int64_t r = (int64_t)(f & 0x1FFFu);        // 13-bit position on the chord
    int64_t y0 = exp2_knot(seg), y1 = exp2_knot(seg + 1);
    int64_t m = y0 + rshr((y1 - y0) * r, 13);  // Q.30 mantissa
    return (int32_t)rshr(m, (int)(14 - n));
}

// e^(x/2^16) in Q.16 for -2^31 <= x <= 0.
__device__ __forceinline__ int32_t nau_exp(int64_t x) {
    return nau_exp2(rshr(x * kLog2eQ30, 30));
}

// SoftPlus in Q.16: e^-|x| + max(x, 0) (Eq. (5) for x <= 0, the symmetry above).
__device__ __forceinline__ int32_t nau_softplus(int32_t x) {
    int64_t xa = x < 0 ? -(int64_t)x : (int64_t)x;
    int64_t e = nau_exp(-xa);
    return sat32(e + (x > 0 ? (int64_t)x : 0));
}

// SiLU in Q.16: for x <= 0, sigma = floor(E*2^16 / (2^16 + E)), E = e^x,
// SiLU = rshr(x * sigma, 16); for x > 0, x + SiLU(-x).
__device__ __forceinline__ int32_t nau_silu(int32_t x) {
    int64_t xn = x < 0 ? (int64_t)x : -(int64_t)x;   // -|x|
    uint32_t e = (uint32_t)nau_exp(xn);             // [0, 2^16]
    uint32_t sig = (e >= 65536u) ? 32768u : ((e << 16) / (65536u + e));
    int64_t sn = rshr(xn * (int64_t)sig, 16);
    return (int32_t)(x > 0 ? (int64_t)x + sn : sn);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ float wave_max_f32(float v) {
    for (int k = 32; k >= 1; k >>= 1) v = fmaxf(v, __shfl_xor(v, k, 64));
    return v;
}
__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
    for (int k = 32; k >= 1; k >>= 1) {
        int32_t o = __shfl_xor(v, k, 64);
        v = o > v ? o : v;
    }
    return v;
}

// non-negative float maxima accumulate as their bit patterns (order-preserving)
__device__ __forceinline__ void atomic_max_nonneg_f32(float* addr, float v) {
    atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace fm
