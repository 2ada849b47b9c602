// Power-of-two quantized causal depthwise conv1d + SiLU + x/B/C requantization.
//
// Review page of FastMamba: the abstract and "What carries the argument"
// (fine-grained power-of-two quantization of the convolution, rescaling by
// shifts); Fig. 2 (conv1d then SiLU in the Mamba2 block).  SiLU goes through
// the 2^v approximation unit (fm_device.hpp).
//
// Thread per (channel, run of kConvTL time steps): the 4-tap window slides in
// registers, so each input is read once; a wave covers 64 consecutive
// channels, so every load and store is coalesced.  d_inner and d_state are
// multiples of 64, so a wave never straddles the x | B | C split.
//
// Dynamic exponents need the maximum of each part over the whole tensor
// before any code is formed, so a second pass writes the codes.  Between the
// passes each wave's 64 x 16 SiLU values s (Q.16) are held as 16-bit words
// T = floor(s * 2^(e - 15)) at the wave's own exponent e (the exponent rule
// applied to the wave's maximum, 24 for an all-zero wave), so |T| <= 255.
// The tensor's exponent p is never above e, and with k = e - p + 1 >= 1,
// rshr(T, k) = floor(s * 2^(p - 16) + 1/2) = rshr(s, 16 - p) exactly (the
// discarded low bits of s are a fraction below one step of T, which cannot
// carry the half-up rounding across an integer).  Runs that record
// quantization statistics keep the 32-bit values, which the statistics need.
#include "fm_internal.hpp"

namespace fm {

constexpr int kConvTL = 16;      // time steps per thread
constexpr int kConvThreads = 256;

struct ConvKParams {
    ConvArgs a;
    int ch;
    int dynamic;
};

// The per-wave exponents of the 16-bit form, after its [T, ch] words in s16.
// Wave blocks are numbered (batch, 16-step block of the sequence, 64-channel
// group), with ceil(len / 64) * 4 step blocks per sequence.
__device__ __forceinline__ int8_t* conv_pblk(const ConvArgs& A, int ch) {
    return reinterpret_cast<int8_t*>(A.s16) + 2 * A.batch * A.len * (int64_t)ch;
}

// One thread: channel c, steps t0 .. t0+n-1 (n = kConvTL unless kTail).
// Dynamic: writes Q.16 SiLU outputs + per-part maxima.  Static: writes codes.
// Dynamic without statistics: the values are held in sv for the wave's
// exponent instead of being written.
template <bool kTail, bool kDyn, bool kXq, bool kStats>
__device__ __forceinline__ void conv_run_steps(const ConvKParams& K, const NauLds& tab, int c,
                                               int64_t row0, int64_t t0, int n, int p_c,
                                               int part, int32_t& amax, float& xmax,
                                               QStat& sx, QStat& sp, int32_t (&sv_hold)[kConvTL]) {
    constexpr bool kHold = kDyn && !kStats;
    const ConvArgs& A = K.a;
    const int di = (int)A.d_inner, N = (int)A.dstate;
    const float qscale = ldexpf(1.0f, p_c);
    const int32_t w0 = A.w_q[c * 4 + 0], w1 = A.w_q[c * 4 + 1], w2 = A.w_q[c * 4 + 2],
                  w3 = A.w_q[c * 4 + 3];
    // a = sat32(rshr(acc, sh) + bias): acc * 2^-sh is exact in float64 (|acc| < 2^17)
    const double ascale = __builtin_ldexp(1.0, 16 - p_c - A.p_w[c]);
    const double bias = (double)A.b_q16[c];
    const float* xrow = A.xbc + row0 * A.xbc_stride + c;  // step t0
    const uint32_t xs = (uint32_t)A.xbc_stride;
    // every load of the run issued up front (3 window inputs + the new ones)
    float win[3];
    float xv[kConvTL];
#pragma unroll
    for (int j = 0; j < 3; ++j) win[j] = t0 > 0 ? xrow[-(int64_t)(3 - j) * A.xbc_stride] : 0.0f;
#pragma unroll
    for (int i = 0; i < kConvTL; ++i) xv[i] = (!kTail || i < n) ? xrow[(uint32_t)i * xs] : 0.0f;
    int32_t xm3, xm2, xm1;  // codes at t-3, t-2, t-1
    if (t0 == 0) {
        if (A.state_in) {
            const int8_t* st = A.state_in + (row0 / A.len * K.ch + c) * 3;
            xm3 = st[0];
            xm2 = st[1];
            xm1 = st[2];
        } else {
            xm3 = xm2 = xm1 = 0;
        }
    } else {  // t0 >= kConvTL >= 3: the window lies inside this call's input
        xm3 = quant_xbc(win[0], qscale);
        xm2 = quant_xbc(win[1], qscale);
        xm1 = quant_xbc(win[2], qscale);
    }
    // outputs of this thread: element (row0 + i, c) of [rows, ch] / of the part
    const int p_part = kDyn ? 0 : A.p_fixed[1 + part];
    const double oscale = __builtin_ldexp(1.0, p_part - 16);
    int32_t* s16 = kDyn && !kHold ? A.s16 + row0 * K.ch + c : nullptr;
    int8_t* code = nullptr;
    uint32_t cstride = 0;
    if (!kDyn) {
        if (part == 0) code = A.x_out + row0 * di + c, cstride = (uint32_t)di;
        else if (part == 1) code = A.b_out + row0 * N + (c - di), cstride = (uint32_t)N;
        else code = A.c_out + row0 * N + (c - di - N), cstride = (uint32_t)N;
    }
    int8_t* xq_out = kXq ? A.xbc_q + row0 * K.ch + c : nullptr;
#pragma unroll
    for (int i = 0; i < kConvTL; ++i) {
        if (kTail && i >= n) continue;
        const float xv_i = xv[i];
        xmax = fmaxf(xmax, fabsf(xv_i));
        const int32_t xq = quant_xbc(xv_i, qscale);
        if constexpr (kStats)
            sx.add((double)xv_i, (double)xq, __builtin_ldexp(1.0, -p_c),
                   fabsf(rintf(xv_i * qscale)) > 127.0f);
        if constexpr (kXq) xq_out[(uint32_t)i * (uint32_t)K.ch] = (int8_t)xq;
        // int8 x int8 products: 24-bit multiplies (full rate; 32-bit ones are not)
        const int32_t acc = __mul24(w0, xm3) + __mul24(w1, xm2) + __mul24(w2, xm1) + __mul24(w3, xq);
        const double a = round_sat_d(__builtin_fma((double)acc, ascale, bias));
        const int32_t sv = (int32_t)nau_silu_d(a, tab);
        const int32_t sa = sv < 0 ? -sv : sv;
        amax = sa > amax ? sa : amax;
        if constexpr (kHold) {
            sv_hold[i] = sv;
        } else if constexpr (kDyn) {
            s16[(uint32_t)i * (uint32_t)K.ch] = sv;
        } else {
            // sat8(rshr(sv, 16 - p_part)): sv * 2^(p_part-16) is exact in float64
            const double q = __builtin_floor(__builtin_fma((double)sv, oscale, 0.5));
            const double qc = __builtin_fmin(__builtin_fmax(q, -127.0), 127.0);
            code[(uint32_t)i * cstride] = (int8_t)qc;
            if constexpr (kStats)
                sp.add((double)sv * 0x1p-16, qc, __builtin_ldexp(1.0, -p_part),
                       __builtin_fabs(q) > 127.0);
        }
        xm3 = xm2;
        xm2 = xm1;
        xm1 = xq;
    }
    if (A.state_out && t0 + n == A.len) {
        int8_t* st = A.state_out + (row0 / A.len * K.ch + c) * 3;
        st[0] = (int8_t)xm3;
        st[1] = (int8_t)xm2;
        st[2] = (int8_t)xm1;
    }
}

template <bool kDyn, bool kStats>
__global__ __launch_bounds__(kConvThreads) void conv_silu_kernel(ConvKParams K) {
    const ConvArgs& A = K.a;
    __shared__ NauLds tab;
    __shared__ float xa_s;  // dynamic: max |xBC|, reduced from its slots by wave 0
    nau_lds_init(tab);
    if (kDyn && (int)blockIdx.x != K.ch / 64 && threadIdx.x < 64) {
        const float v = __int_as_float(slots_wave_max(A.xbc_amax_slots));
        if (threadIdx.x == 0) {
            xa_s = v;
            if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) *A.xbc_amax = v;
        }
    }
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if ((int)blockIdx.x == K.ch / 64) {
        // the extra column of workgroups: dt and the decay for the (token, head)
        // pairs of this workgroup's steps, as the scan's prologue forms them
        // 32-bit indices inside the workgroup (at most 64 steps x nheads pairs)
        const int64_t L = A.len;
        const int H = (int)A.nheads;
        const int64_t t0 = (int64_t)blockIdx.y * (kConvThreads / 64) * kConvTL;
        const int nt = (int)(L - t0 < (kConvThreads / 64) * kConvTL ? L - t0
                                                                    : (kConvThreads / 64) * kConvTL);
        const int64_t row0 = (int64_t)blockIdx.z * L + t0;
        constexpr int kB = 8;  // pairs per thread whose loads go out together
        for (int i0 = threadIdx.x; i0 < nt * H; i0 += kB * kConvThreads) {
            float raw[kB], bias[kB];
            int32_t aq[kB];
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int i = i0 + k * kConvThreads;
                const int ti = i / H, h = i - ti * H;
                const bool ok = i < nt * H;
                raw[k] = ok ? A.dt_raw[(row0 + ti) * A.dt_stride + h] : 0.0f;
                bias[k] = ok ? A.dt_bias[h] : 0.0f;
                aq[k] = ok ? A.a_q16[h] : 0;
            }
#pragma unroll
            for (int k = 0; k < kB; ++k) {
                const int i = i0 + k * kConvThreads;
                if (i >= nt * H) break;
                const int ti = i / H, h = i - ti * H;
                const int64_t row = row0 + ti;
                const int32_t dt = nau_softplus_f(f2i_sat(rintf((raw[k] + bias[k]) * 65536.0f)), tab);
                A.dt_out[row * H + h] = dt;
                A.da_out[row * H + h] = nau_exp_f(sat32(rshr((int64_t)dt * (int64_t)aq[k], 16)), tab);
            }
        }
        return;
    }
    const int p_c = kDyn ? pot_from_f32(xa_s) : A.p_fixed[0];
    if (!kDyn && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < 4)
        A.p_out[threadIdx.x] = A.p_fixed[threadIdx.x];
    const int c0 = blockIdx.x * 64;  // a wave covers 64 channels of one part
    const int c = c0 + lane;
    const int di = (int)A.d_inner, N = (int)A.dstate;
    const int part = c0 < di ? 0 : (c0 < di + N ? 1 : 2);
    const int64_t L = A.len;
    const int64_t t0 = ((int64_t)blockIdx.y * (kConvThreads / 64) + wave) * kConvTL;
    if (t0 >= L) return;  // whole wave: no barrier follows
    const int64_t row0 = (int64_t)blockIdx.z * L + t0;
    const int n = (int)(t0 + kConvTL < L ? kConvTL : L - t0);
    int32_t amax = 0;
    float xmax = 0.0f;
    QStat sx, sp;
    int32_t sv[kConvTL];
    if (A.xbc_q) {
        if (n == kConvTL) conv_run_steps<false, kDyn, true, kStats>(K, tab, c, row0, t0, n, p_c, part, amax, xmax, sx, sp, sv);
        else conv_run_steps<true, kDyn, true, kStats>(K, tab, c, row0, t0, n, p_c, part, amax, xmax, sx, sp, sv);
    } else {
        if (n == kConvTL) conv_run_steps<false, kDyn, false, kStats>(K, tab, c, row0, t0, n, p_c, part, amax, xmax, sx, sp, sv);
        else conv_run_steps<true, kDyn, false, kStats>(K, tab, c, row0, t0, n, p_c, part, amax, xmax, sx, sp, sv);
    }
    if constexpr (kStats) {  // every lane of the wave is here (one part per wave)
        qstat_flush(sx, A.qs, FM_QP_XBC);
        if (!kDyn) qstat_flush(sp, A.qs, FM_QP_X + part);
    }
    // per-wave maxima (all lanes of a wave are in one part); dynamic: into a slot
    // of the part's region, by the wave's time block
    amax = wave_max_i32(amax);
    xmax = wave_max_f32(xmax);
    const int64_t tb = (int64_t)blockIdx.z * gridDim.y * (kConvThreads / 64) +
                       (int64_t)blockIdx.y * (kConvThreads / 64) + wave;
    if constexpr (kDyn && !kStats) {
        // the wave's values as 16-bit words at the wave's exponent, the exponent
        // in the table after them (one byte per wave block: 16 steps x 64 channels)
        const int e = amax == 0 ? kPMax : pot_from_q16(amax);
        int16_t* out = reinterpret_cast<int16_t*>(A.s16) + row0 * K.ch + c;
        // floor(v * 2^(e - 15)): e <= 24, so a left shift moves at most 9 bits
        // (|result| <= 255); right shifts floor, 31 places at most
        const int ls = e >= 15 ? e - 15 : 0, rs = e >= 15 ? 0 : (15 - e < 31 ? 15 - e : 31);
        auto word = [&](int i) { return (int16_t)((sv[i] << ls) >> rs); };
        if (n == kConvTL) {
#pragma unroll
            for (int i = 0; i < kConvTL; ++i) out[(uint32_t)i * (uint32_t)K.ch] = word(i);
        } else {
#pragma unroll
            for (int i = 0; i < kConvTL; ++i)
                if (i < n) out[(uint32_t)i * (uint32_t)K.ch] = word(i);
        }
        if (lane == 0)
            conv_pblk(A, K.ch)[tb * (K.ch / 64) + blockIdx.x] = (int8_t)e;
    }
    if (lane == 0) {
        if (kDyn) {
            slot_max(A.amax_slots + part * kSlotRegionWords, tb, amax);
        } else if (A.amax_stats) {
            if (amax > 0) atomic_max_i32(&A.amax_stats[1 + part], amax);
            if (xmax > 0.0f) atomic_max_nonneg_f32((float*)&A.amax_stats[0], xmax);
        }
    }
}

// Dynamic second pass: exponents from the maxima, SiLU values -> int8 codes
// (k16: from the 16-bit words and their wave exponents; otherwise from the
// 32-bit Q.16 values, with statistics).
// grid.y = token row, threads over groups of kRqCh channels (one 16-byte load
// per row: 8 16-bit words, or 4 32-bit values).
constexpr int kRqRows = 4;  // rows per thread in the requantization pass
template <bool k16> constexpr int kRqCh = k16 ? 8 : 4;

template <bool k16>
__global__ __launch_bounds__(kConvThreads) void requant_kernel(ConvKParams K) {
    const ConvArgs& A = K.a;
    const int di = (int)A.d_inner, N = (int)A.dstate;
    const int c = (blockIdx.x * kConvThreads + threadIdx.x) * kRqCh<k16>;
    const bool active = c < K.ch;  // idle lanes stay for the statistics' wave sums
    const int64_t rows = A.batch * A.len;
    // 16-bit form: the wave block of (row, c) in the exponent table
    const int64_t L = A.len, sblocks = (L + 63) / 64 * (kConvThreads / 64);
    const int8_t* pblk = k16 ? conv_pblk(A, K.ch) + c / 64 : nullptr;
    // kRqRows rows per thread and round, their loads issued before any use (the
    // first round's before the maxima are known)
    int4 sr[kRqRows];
    int32_t eb[kRqRows];
    auto load_round = [&](int64_t r0) {
        // (sequence, step) of row r0, then stepped along the round's rows
        int64_t b = 0, t = 0;
        if constexpr (k16) {
            b = r0 / L;
            t = r0 - b * L;
        }
#pragma unroll
        for (int k = 0; k < kRqRows; ++k) {
            if constexpr (k16) {
                while (t >= L) {
                    t -= L;
                    ++b;
                }
                const bool ok = r0 + k < rows;
                sr[k] = ok ? *reinterpret_cast<const int4*>(
                                 reinterpret_cast<const int16_t*>(A.s16) + (r0 + k) * K.ch + c)
                           : make_int4(0, 0, 0, 0);
                eb[k] = ok ? pblk[(b * sblocks + t / kConvTL) * (K.ch / 64)] : kPMax;
                ++t;
            } else {
                sr[k] = r0 + k < rows ? *reinterpret_cast<const int4*>(A.s16 + (r0 + k) * K.ch + c)
                                      : make_int4(0, 0, 0, 0);
            }
        }
    };
    const int64_t rfirst = (int64_t)blockIdx.y * kRqRows;
    if (active) load_round(rfirst);
    // the part maxima from the conv pass's slot regions: wave 0 reduces, LDS shares
    __shared__ int32_t pm_s[3];
    if (threadIdx.x < 64) {
#pragma unroll
        for (int i = 0; i < 3; ++i) {
            const int32_t v = slots_wave_max(A.amax_slots + i * kSlotRegionWords);
            if (threadIdx.x == 0) pm_s[i] = v;
        }
    }
    __syncthreads();
    const int32_t pm[3] = {pm_s[0], pm_s[1], pm_s[2]};
    if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
        A.p_out[0] = pot_from_f32(*A.xbc_amax);
        for (int i = 0; i < 3; ++i) {
            A.amax_q16[i] = pm[i];
            A.p_out[1 + i] = pot_from_q16(pm[i]);
        }
        if (A.amax_stats) {
            atomicMax((unsigned int*)&A.amax_stats[0], __float_as_uint(*A.xbc_amax));
            for (int i = 0; i < 3; ++i) atomicMax(&A.amax_stats[1 + i], pm[i]);
        }
    }
    const int part = !active ? 0 : (c < di ? 0 : (c < di + N ? 1 : 2));
    const int32_t amax_part = part == 0 ? pm[0] : (part == 1 ? pm[1] : pm[2]);
    // sat8(rshr(s, 16 - p)): s * 2^(p-16) + 1/2 is exact in float64 for every
    // p in [-24, 24] (|s| < 2^31), so floor gives rshr's value, shifts up included
    const double sc = __builtin_ldexp(1.0, pot_from_q16(amax_part) - 16);
    auto q8 = [&](int32_t v) {
        const double q = __builtin_floor(__builtin_fma((double)v, sc, 0.5));
        return (signed char)__builtin_fmin(__builtin_fmax(q, -127.0), 127.0);
    };
    // 16-bit words T at the wave exponent e: code = sat8(rshr(T, e - p + 1)), where
    // e - p + 1 >= 1 and shifts past 16 leave 0 (|T| <= 255)
    const int p_part = pot_from_q16(amax_part);
    auto q8w = [&](int32_t t, int32_t e) {
        const int k = e - p_part + 1;
        const int32_t r = k > 16 ? 0 : (t + (1 << (k - 1))) >> k;
        return (signed char)(r < -127 ? -127 : (r > 127 ? 127 : r));
    };
    QStat st;
    const double step = __builtin_ldexp(1.0, 16 - pot_from_q16(amax_part));
    for (int64_t r0 = rfirst; active && r0 < rows; r0 += (int64_t)gridDim.y * kRqRows) {
        if (r0 != rfirst) load_round(r0);
#pragma unroll
        for (int k = 0; k < kRqRows; ++k) {
            const int64_t row = r0 + k;
            if (row >= rows) break;
            const int4 s = sr[k];
            char4 q;
            if constexpr (k16) {
                // eight words -> eight codes, stored as one 8-byte word
                const int32_t e = eb[k];
                const int32_t wd[4] = {s.x, s.y, s.z, s.w};
                uint32_t out[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    char4 o;
                    o.x = q8w((int16_t)(wd[2 * h] & 0xFFFF), e);
                    o.y = q8w((int16_t)(wd[2 * h] >> 16), e);
                    o.z = q8w((int16_t)(wd[2 * h + 1] & 0xFFFF), e);
                    o.w = q8w((int16_t)(wd[2 * h + 1] >> 16), e);
                    out[h] = __builtin_bit_cast(uint32_t, o);
                }
                const uint2 o8 = make_uint2(out[0], out[1]);
                if (part == 0) *reinterpret_cast<uint2*>(A.x_out + row * di + c) = o8;
                else if (part == 1) *reinterpret_cast<uint2*>(A.b_out + row * N + (c - di)) = o8;
                else *reinterpret_cast<uint2*>(A.c_out + row * N + (c - di - N)) = o8;
                continue;
            } else {
                q.x = q8(s.x);
                q.y = q8(s.y);
                q.z = q8(s.z);
                q.w = q8(s.w);
            }
            if (!k16 && A.qs) {
                const int32_t sv[4] = {s.x, s.y, s.z, s.w};
                const signed char qc[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const double qr = __builtin_floor(__builtin_fma((double)sv[e], sc, 0.5));
                    st.add((double)sv[e] * 0x1p-16, (double)qc[e], step * 0x1p-16,
                           __builtin_fabs(qr) > 127.0);
                }
            }
            if (part == 0) *reinterpret_cast<char4*>(A.x_out + row * di + c) = q;
            else if (part == 1) *reinterpret_cast<char4*>(A.b_out + row * N + (c - di)) = q;
            else *reinterpret_cast<char4*>(A.c_out + row * N + (c - di - N)) = q;
        }
    }
    if (!k16 && A.qs)  // a wave may span two parts: one wave sum per part
        for (int pt = 0; pt < 3; ++pt)
            qstat_flush(part == pt && active ? st : QStat{}, A.qs, FM_QP_X + pt);
}

__global__ __launch_bounds__(256) void amax_strided_kernel(const float* __restrict__ x, int64_t rows,
                                                           int64_t cols, int64_t stride,
                                                           int32_t* amax_slots) {
    float m = 0.0f;
    const int64_t total = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i - r * cols;
        m = fmaxf(m, fabsf(x[r * stride + c]));
    }
    m = wave_max_f32(m);
    if ((threadIdx.x & 63) == 0)
        slot_max(amax_slots, (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6), (int32_t)__float_as_uint(m));
}

fm_status amax_strided_run(const float* x, int64_t rows, int64_t cols, int64_t stride,
                           int32_t* amax_slots, hipStream_t s) {
    int64_t total = rows * cols;
    int g = (int)((total + 255) / 256);
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    amax_strided_kernel<<<g, 256, 0, s>>>(x, rows, cols, stride, amax_slots);
    return check_launch("amax_strided_kernel");
}

fm_status conv_run(const ConvArgs& a, hipStream_t s) {
    ConvKParams K{a, (int)(a.d_inner + 2 * a.dstate), a.p_fixed == nullptr ? 1 : 0};
    const int64_t per_block = (kConvThreads / 64) * kConvTL;
    dim3 grid((unsigned)(K.ch / 64 + (a.dt_raw ? 1 : 0)),
              (unsigned)((a.len + per_block - 1) / per_block), (unsigned)a.batch);
    if (a.qs) {  // statistics of the quantization points: a separate instance
        if (K.dynamic) conv_silu_kernel<true, true><<<grid, kConvThreads, 0, s>>>(K);
        else conv_silu_kernel<false, true><<<grid, kConvThreads, 0, s>>>(K);
    } else {
        if (K.dynamic) conv_silu_kernel<true, false><<<grid, kConvThreads, 0, s>>>(K);
        else conv_silu_kernel<false, false><<<grid, kConvThreads, 0, s>>>(K);
    }
    fm_status st = check_launch("conv_silu_kernel");
    if (st != FM_OK || !K.dynamic) return st;
    const int64_t rows = a.batch * a.len, rblocks = (rows + kRqRows - 1) / kRqRows;
    auto rgrid = [&](int per) {
        return dim3((unsigned)((K.ch / per + kConvThreads - 1) / kConvThreads),
                    (unsigned)(rblocks < 65535 ? rblocks : 65535));
    };
    if (a.qs) requant_kernel<false><<<rgrid(kRqCh<false>), kConvThreads, 0, s>>>(K);
    else requant_kernel<true><<<rgrid(kRqCh<true>), kConvThreads, 0, s>>>(K);
    return check_launch("requant_kernel");
}

}  // namespace fm
