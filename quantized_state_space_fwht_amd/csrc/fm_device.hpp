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

#include "fm.h"

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
// With a = m * 2^e, m in [0.5, 1): p = 7 - e when m * 128 <= 127, else 6 - e.
__device__ __forceinline__ int pot_from_f32(float a) {
    if (!(a > 0.0f)) return 0;
    int e;
    const float m = frexpf(a, &e);
    int p = (m <= 0.9921875f) ? 7 - e : 6 - e;
    return p > kPMax ? kPMax : (p < kPMin ? kPMin : p);
}

// Largest p in [kPMin, kPMax] with (m / 2^16) * 2^p <= 127 for a Q.16 maximum m >= 0.
// For m in [2^(k-1), 2^k) every p >= 24 - k fails, so the search starts there.
__device__ __forceinline__ int pot_from_q16(int64_t m) {
    if (m <= 0) return 0;
    const int k = 64 - __clzll((unsigned long long)m);
    const int64_t lim = (int64_t)127 << 16;
    int p0 = 24 - k;
    if (p0 > kPMax) p0 = kPMax;
    for (int p = p0; p > kPMin; --p) {
        const bool ok = p >= 0 ? ((m << p) <= lim) : (m <= (lim << (-p)));
        if (ok) return p;
    }
    return kPMin;
}

// xBC -> int8 code with its power-of-two scale 2^p_c: sat8(rint(v * 2^p_c))
__device__ __forceinline__ int32_t quant_xbc(float v, float scale) {
    return (int32_t)fminf(fmaxf(rintf(v * scale), -127.0f), 127.0f);
}

// clamp(floor(v + 1/2)) to the int32 range for an integer-valued or half-step
// v, as float64 and as int32
__device__ __forceinline__ double round_sat_d(double v) {
    return __builtin_fmin(__builtin_fmax(__builtin_floor(v + 0.5), -2147483648.0), 2147483647.0);
}

__device__ __forceinline__ int32_t round_sat32(double v) { return (int32_t)round_sat_d(v); }

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

// ---------------------------------------------------------------- NAU evaluation
// Integer definitions (Q.16 in and out):
//   2^(v/2^16), v <= 0:  n = v >> 16, f = v & 0xFFFF, seg = f >> 13, r = f & 0x1FFF,
//                        m = Y[seg] + rshr((Y[seg+1] - Y[seg]) * r, 13),  result rshr(m, 14 - n)
//   e^(x/2^16), x <= 0:  2^(rshr(x * kLog2eQ30, 30) / 2^16)
// They are evaluated with float64 operations on integer-valued operands (full
// vector rate on MI355X, where 64-bit integer multiplies and shifts are not).
// Every product below stays under 2^53 wherever the result is not already
// known to be 0, so each floor() sees the exact rational value and the results
// equal the integer definitions.  The chords live in LDS as pairs
// (Y[i], (Y[i+1] - Y[i]) * 2^-13), one 16-byte read per evaluation
// (nau_lds_init or nau_lds_set, then a barrier before first use).
struct NauLds {
    struct alignas(16) Chord {
        double y, d;
    } c[8];
};

__device__ __forceinline__ void nau_lds_set(NauLds& t, int i, int64_t y0, int64_t y1) {
    t.c[i].y = (double)y0;
    t.c[i].d = (double)(y1 - y0) * 0x1p-13;  // exact: |y1 - y0| < 2^53
}

__device__ __forceinline__ void nau_lds_init(NauLds& t) {
    if (threadIdx.x < 8) nau_lds_set(t, threadIdx.x, exp2_knot(threadIdx.x), exp2_knot(threadIdx.x + 1));
}

// 2^(v/2^16) in Q.16 for an integer-valued vf in [-18*2^16, 0].  Below
// v = -18*2^16 the Q.30 mantissa is shifted right by >= 32 and rounds to 0.
__device__ __forceinline__ double nau_exp2_d(double vf, const NauLds& t) {
    const int v = (int)vf;
    const int n = v >> 16;  // -18..0
    const int seg = (v >> 13) & 7;
    const double r = (double)(v & 0x1FFF);
    const NauLds::Chord ch = t.c[seg];
    // m = Y[seg] + rshr((Y[seg+1] - Y[seg]) * r, 13): the product is below 2^41
    const double m = ch.y + __builtin_floor(__builtin_fma(ch.d, r, 0.5));
    // rshr(m, 14 - n): m * 2^(n-14) + 1/2 spans at most 50 bits
    return __builtin_floor(__builtin_ldexp(m, n - 14) + 0.5);
}

// e^(x/2^16) in Q.16 for an integer-valued xd in [-2^31, 0].  The argument
// v = rshr(x * kLog2eQ30, 30) is exact while |x| < 2^22 (x * kLog2eQ30 < 2^53);
// beyond, v lies far below the clamp at -18*2^16 whatever the rounding.
__device__ __forceinline__ double nau_exp_d(double xd, const NauLds& t) {
    constexpr double kL = (double)kLog2eQ30 * 0x1p-30;  // exact
    const double vf = __builtin_fmax(__builtin_floor(__builtin_fma(xd, kL, 0.5)), -1179648.0);
    return nau_exp2_d(vf, t);
}

// e^(x/2^16) in Q.16; arguments > 0 (outside the unit's domain) are taken as 0.
__device__ __forceinline__ int32_t nau_exp_f(int32_t x, const NauLds& t) {
    return (int32_t)nau_exp_d(__builtin_fmin((double)x, 0.0), t);
}

// SoftPlus in Q.16: e^-|x| + max(x, 0) (Eq. (5) for x <= 0, the symmetry above).
__device__ __forceinline__ int32_t nau_softplus_f(int32_t x, const NauLds& t) {
    const double xd = (double)x;
    const double e = nau_exp_d(-__builtin_fabs(xd), t);
    return (int32_t)__builtin_fmin(e + __builtin_fmax(xd, 0.0), 2147483647.0);  // sat32
}

// SiLU in Q.16 of an integer-valued xd in [-2^31, 2^31) (as float64): for
// x <= 0, sigma = floor(E*2^16 / (2^16 + E)), E = e^x, SiLU = rshr(x * sigma, 16);
// for x > 0, x + SiLU(-x).  The quotient is E / b with b = 1 + E*2^-16 in
// [1, 2]: the hardware reciprocal of b (relative error near 2^-23) refined by
// one Newton step is within 2^-44 of 1/b, so E / b + 2^-20 lies at or above the
// quotient and below the next integer, whose distance from it is at least
// 1 / (2^16 + E) >= 2^-17; floor() gives sigma.  E = 2^16 gives 2^15.
__device__ __forceinline__ double nau_silu_d(double xd, const NauLds& t) {
    const double xn = -__builtin_fabs(xd);
    const double e = nau_exp_d(xn, t);  // [0, 2^16]
    const double b = __builtin_fma(e, 0x1p-16, 1.0);
    const double r0 = __builtin_amdgcn_rcp(b);
    const double r1 = __builtin_fma(r0, __builtin_fma(-b, r0, 1.0), r0);
    const double sig = __builtin_floor(__builtin_fma(e, r1, 0x1p-20));
    // rshr(xn * sigma, 16): |xn * sigma| < 2^46
    const double sn = __builtin_floor(__builtin_fma(xn * 0x1p-16, sig, 0.5));
    return sn + __builtin_fmax(xd, 0.0);
}

__device__ __forceinline__ int32_t nau_silu_f(int32_t x, const NauLds& t) {
    return (int32_t)nau_silu_d((double)x, t);
}

// rint()ed float32 -> int32 with saturation, as an integer-valued float64
__device__ __forceinline__ double f2d_sat(float f) {
    return __builtin_fmin(__builtin_fmax((double)f, -2147483648.0), 2147483647.0);
}

// ---------------------------------------------------------------- 256-point FWHT
// H_256 / 16 of one 256-block held 4 values per lane (lane l: elements 4l..4l+3).
// Stages h = 1, 2 inside the lane, then h = 4m with the partner lane l ^ m: the
// lane with bit m clear keeps a + b, its partner a - b.  fma(+-1, v, p) rounds
// exactly like the plain sum or difference, so every lane runs one instruction
// stream.  The final 1/16 is exact.
__device__ __forceinline__ float4 fwht256_lane(float4 v, int lane) {
    float t0 = v.x + v.y, t1 = v.x - v.y, t2 = v.z + v.w, t3 = v.z - v.w;
    v.x = t0 + t2;
    v.z = t0 - t2;
    v.y = t1 + t3;
    v.w = t1 - t3;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float px = __shfl_xor(v.x, m, 64);
        const float py = __shfl_xor(v.y, m, 64);
        const float pz = __shfl_xor(v.z, m, 64);
        const float pw = __shfl_xor(v.w, m, 64);
        const float sg = (lane & m) ? -1.0f : 1.0f;
        v.x = __builtin_fmaf(sg, v.x, px);
        v.y = __builtin_fmaf(sg, v.y, py);
        v.z = __builtin_fmaf(sg, v.z, pz);
        v.w = __builtin_fmaf(sg, v.w, pw);
    }
    v.x *= 0.0625f;
    v.y *= 0.0625f;
    v.z *= 0.0625f;
    v.w *= 0.0625f;
    return v;
}

__device__ __forceinline__ float absmax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// q = sat8(rint(v * c)) for four elements, packed in memory order (byte i =
// element i).  The product is clamped to [-127, 127] first (rint and the clamp
// commute there: a product in (127, 127.5] rounds to 127 either way), then
// adding 1.5 * 2^23 rounds it to an integer, ties to even as rint does, and
// leaves that integer in the low byte of the sum's bit pattern (two's
// complement: the sum is 0x4B400000 + q).  Three byte permutes pack the codes.
__device__ __forceinline__ uint32_t quant_pack4(float4 v, float c) {
    constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
    const uint32_t a = __float_as_uint(fminf(fmaxf(v.x * c, -127.0f), 127.0f) + kMagic);
    const uint32_t b = __float_as_uint(fminf(fmaxf(v.y * c, -127.0f), 127.0f) + kMagic);
    const uint32_t d = __float_as_uint(fminf(fmaxf(v.z * c, -127.0f), 127.0f) + kMagic);
    const uint32_t e = __float_as_uint(fminf(fmaxf(v.w * c, -127.0f), 127.0f) + kMagic);
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a.b0, b.b0
    const uint32_t de = __builtin_amdgcn_perm(e, d, 0x0c0c0400u);  // d.b0, e.b0
    return __builtin_amdgcn_perm(de, ab, 0x05040100u);
}

// q = sat8(rint(v * c)) per element
__device__ __forceinline__ char4 quant4(float4 v, float c) {
    return __builtin_bit_cast(char4, quant_pack4(v, c));
}

// sum of a per-lane partial over the wave in the fixed xor order k = 32, 16, .., 1
__device__ __forceinline__ float wave_sum_fixed(float a) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) a = a + __shfl_xor(a, k, 64);
    return a;
}

// ---------------------------------------------------------------- quantization statistics
// Per-thread accumulator of one quantization point (fm_quant_stats), flushed
// once per wave: wave sums, then one set of atomics from lane 0.
struct QStat {
    uint32_t n = 0, clip = 0;
    double se = 0.0, sv = 0.0;
    __device__ __forceinline__ void add(double v, double q, double step, bool clipped) {
        const double e = v - q * step;
        n += 1;
        clip += clipped ? 1u : 0u;
        se = __builtin_fma(e, e, se);
        sv = __builtin_fma(v, v, sv);
    }
};

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

// Slotted grid maxima.  A region is kSlots words kSlotStride words (256 bytes)
// apart, zeroed before the producing launch.  Producers add their value to one
// slot, chosen by a key (a block or wave index), with an atomic max that
// returns nothing; consumers reduce the slots with one load per lane.  Atomics
// and coherent reads of one cache line from thousands of waves serialize at
// the memory side; spread over 32 lines they do not.  Values are non-negative
// (magnitudes, or the bit patterns of non-negative floats, which order alike).
constexpr int kSlots = 32;
constexpr int kSlotStride = 64;
constexpr int kSlotRegionWords = kSlots * kSlotStride;

__device__ __forceinline__ void slot_max(int32_t* region, int64_t key, int32_t v) {
    if (v > 0) atomicMax(region + (int)(key % kSlots) * kSlotStride, v);
}
// every lane of the wave must call it
__device__ __forceinline__ int32_t slots_wave_max(const int32_t* region) {
    const int lane = threadIdx.x & 63;
    return wave_max_i32(lane < kSlots ? region[lane * kSlotStride] : 0);
}

// Maxima shared by a whole grid.  The stored value only grows, so the atomic
// is skipped when a plain (device-coherent) read already covers v: a stale
// read can only cost an extra atomic, never lose one.  Thousands of waves
// updating one word would otherwise serialize on it.
__device__ __forceinline__ void atomic_max_i32(int32_t* addr, int32_t v) {
    if (__hip_atomic_load(addr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < v) atomicMax(addr, v);
}
// non-negative float maxima accumulate as their bit patterns (order-preserving)
__device__ __forceinline__ void atomic_max_nonneg_f32(float* addr, float v) {
    unsigned int* a = reinterpret_cast<unsigned int*>(addr);
    const unsigned int u = __float_as_uint(v);
    if (__hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < u) atomicMax(a, u);
}

// statistics of four Hadamard-point elements quantized with coefficient c
// (code = sat8(rint(v * c)), dequant scale s_dq = 1 / c)
__device__ __forceinline__ void quant_stat4(QStat& st, float4 v, float c, float s_dq) {
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float r = rintf(e[i] * c);
        st.add((double)e[i], (double)fminf(fmaxf(r, -127.0f), 127.0f), (double)s_dq,
               fabsf(r) > 127.0f);
    }
}

// wave sum of the accumulator, then lane 0 adds it into point `pt` of qs
__device__ inline void qstat_flush(QStat a, fm_quant_stats* qs, int pt) {
    for (int k = 32; k >= 1; k >>= 1) {
        a.n += __shfl_xor(a.n, k, 64);
        a.clip += __shfl_xor(a.clip, k, 64);
        a.se += __shfl_xor(a.se, k, 64);
        a.sv += __shfl_xor(a.sv, k, 64);
    }
    if ((threadIdx.x & 63) == 0 && a.n > 0) {
        atomicAdd(&qs->count[pt], (unsigned long long)a.n);
        if (a.clip) atomicAdd(&qs->clipped[pt], (unsigned long long)a.clip);
        atomicAdd(&qs->sq_err[pt], a.se);
        atomicAdd(&qs->sq_val[pt], a.sv);
    }
}

}  // namespace fm
