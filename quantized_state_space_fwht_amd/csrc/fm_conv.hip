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
#include "fm_internal.hpp"

namespace fm {

constexpr int kConvTL = 16;      // time steps per thread
constexpr int kConvThreads = 256;

struct ConvKParams {
    ConvArgs a;
    int ch;
    int dynamic;
};

__device__ __forceinline__ int8_t quant_xbc(float v, float scale) {
    return (int8_t)fminf(fmaxf(rintf(v * scale), -127.0f), 127.0f);
}

// Dynamic: writes Q.16 SiLU outputs + per-part maxima.  Static: writes codes.
__global__ __launch_bounds__(kConvThreads) void conv_silu_kernel(ConvKParams K) {
    const ConvArgs& A = K.a;
    __shared__ int sp[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (threadIdx.x == 0) {
        if (K.dynamic) {
            sp[0] = pot_from_f32(*A.xbc_amax);
            sp[1] = sp[2] = sp[3] = 0;
        } else {
            for (int i = 0; i < 4; ++i) sp[i] = A.p_fixed[i];
        }
        if (!K.dynamic && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
            for (int i = 0; i < 4; ++i) A.p_out[i] = sp[i];
    }
    __syncthreads();
    const int c = blockIdx.x * 64 + lane;
    const int64_t b = blockIdx.z;
    const int64_t L = A.len;
    const int64_t t0 = ((int64_t)blockIdx.y * (kConvThreads / 64) + wave) * kConvTL;
    const int di = (int)A.d_inner, N = (int)A.dstate;
    const int part = c < di ? 0 : (c < di + N ? 1 : 2);
    int32_t amax = 0;
    float xmax = 0.0f;
    if (t0 < L) {
        const int p_c = sp[0];
        const float qscale = ldexpf(1.0f, p_c);
        const int32_t w0 = A.w_q[c * 4 + 0], w1 = A.w_q[c * 4 + 1], w2 = A.w_q[c * 4 + 2],
                      w3 = A.w_q[c * 4 + 3];
        const int sh = p_c + A.p_w[c] - 16;
        const int64_t bias = A.b_q16[c];
        const int p_part = sp[1 + part];
        const float* xrow = A.xbc + (b * L) * A.xbc_stride + c;
        int32_t xm3, xm2, xm1;  // inputs at t-3, t-2, t-1
        if (t0 == 0) {
            if (A.state_in) {
                const int8_t* st = A.state_in + (b * K.ch + c) * 3;
                xm3 = st[0];
                xm2 = st[1];
                xm1 = st[2];
            } else {
                xm3 = xm2 = xm1 = 0;
            }
        } else {  // t0 >= kConvTL >= 3: the window lies inside this call's input
            xm3 = quant_xbc(xrow[(t0 - 3) * A.xbc_stride], qscale);
            xm2 = quant_xbc(xrow[(t0 - 2) * A.xbc_stride], qscale);
            xm1 = quant_xbc(xrow[(t0 - 1) * A.xbc_stride], qscale);
        }
        const int64_t t1 = t0 + kConvTL < L ? t0 + kConvTL : L;
        for (int64_t t = t0; t < t1; ++t) {
            const float xv = xrow[t * A.xbc_stride];
            xmax = fmaxf(xmax, fabsf(xv));
            const int32_t xq = quant_xbc(xv, qscale);
            const int64_t row = b * L + t;
            if (A.xbc_q) A.xbc_q[row * K.ch + c] = (int8_t)xq;
            const int64_t acc = (int64_t)(w0 * xm3 + w1 * xm2 + w2 * xm1 + w3 * xq);
            const int32_t a = sat32(rshr(acc, sh) + bias);
            const int32_t s = nau_silu(a);
            const int32_t sa = s < 0 ? -s : s;
            amax = sa > amax ? sa : amax;
            if (K.dynamic) {
                A.s16[row * K.ch + c] = s;
            } else {
                const int8_t code = sat8(rshr((int64_t)s, 16 - p_part));
                if (part == 0) A.x_out[row * di + c] = code;
                else if (part == 1) A.b_out[row * N + (c - di)] = code;
                else A.c_out[row * N + (c - di - N)] = code;
            }
            xm3 = xm2;
            xm2 = xm1;
            xm1 = xq;
        }
        if (A.state_out && t1 == L) {
            int8_t* st = A.state_out + (b * K.ch + c) * 3;
            st[0] = (int8_t)xm3;
            st[1] = (int8_t)xm2;
            st[2] = (int8_t)xm1;
        }
    }
    // per-wave maxima (all lanes of a wave are in one part)
    amax = wave_max_i32(amax);
    xmax = wave_max_f32(xmax);
    if (lane == 0) {
        if (K.dynamic) {
            if (amax > 0) atomicMax(&A.amax_q16[part], amax);
        } else if (A.amax_stats) {
            if (amax > 0) atomicMax(&A.amax_stats[1 + part], amax);
            if (xmax > 0.0f) atomicMax((unsigned int*)&A.amax_stats[0], __float_as_uint(xmax));
        }
    }
}

// Dynamic second pass: exponents from the maxima, Q.16 -> int8 codes.
__global__ __launch_bounds__(kConvThreads) void requant_kernel(ConvKParams K, int64_t total) {
    const ConvArgs& A = K.a;
    __shared__ int sp[4];
    if (threadIdx.x == 0) {
        sp[0] = pot_from_f32(*A.xbc_amax);
        for (int i = 0; i < 3; ++i) sp[1 + i] = pot_from_q16(A.amax_q16[i]);
        if (blockIdx.x == 0) {
            for (int i = 0; i < 4; ++i) A.p_out[i] = sp[i];
            if (A.amax_stats) {
                atomicMax((unsigned int*)&A.amax_stats[0], __float_as_uint(*A.xbc_amax));
                for (int i = 0; i < 3; ++i) atomicMax(&A.amax_stats[1 + i], A.amax_q16[i]);
            }
        }
    }
    __syncthreads();
    const int di = (int)A.d_inner, N = (int)A.dstate;
    // 4 channels per thread (ch % 64 == 0)
    const int64_t nq = total / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nq;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i * 4;
        const int64_t row = e / K.ch;
        const int c = (int)(e - row * K.ch);
        const int4 s = *reinterpret_cast<const int4*>(A.s16 + e);
        const int part = c < di ? 0 : (c < di + N ? 1 : 2);
        const int sh = 16 - sp[1 + part];
        char4 q;
        q.x = sat8(rshr((int64_t)s.x, sh));
        q.y = sat8(rshr((int64_t)s.y, sh));
        q.z = sat8(rshr((int64_t)s.z, sh));
        q.w = sat8(rshr((int64_t)s.w, sh));
        if (part == 0) *reinterpret_cast<char4*>(A.x_out + row * di + c) = q;
        else if (part == 1) *reinterpret_cast<char4*>(A.b_out + row * N + (c - di)) = q;
        else *reinterpret_cast<char4*>(A.c_out + row * N + (c - di - N)) = q;
    }
}

__global__ __launch_bounds__(256) void amax_strided_kernel(const float* __restrict__ x, int64_t rows,
                                                           int64_t cols, int64_t stride,
                                                           float* amax) {
    float m = 0.0f;
    const int64_t total = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = i / cols, c = i - r * cols;
        m = fmaxf(m, fabsf(x[r * stride + c]));
    }
    m = wave_max_f32(m);
    if ((threadIdx.x & 63) == 0 && m > 0.0f) atomic_max_nonneg_f32(amax, m);
}

fm_status amax_strided_run(const float* x, int64_t rows, int64_t cols, int64_t stride,
                           float* amax, hipStream_t s) {
    int64_t total = rows * cols;
    int g = (int)((total + 255) / 256);
    if (g > 2048) g = 2048;
    if (g < 1) g = 1;
    amax_strided_kernel<<<g, 256, 0, s>>>(x, rows, cols, stride, amax);
    return check_launch("amax_strided_kernel");
}

fm_status conv_run(const ConvArgs& a, hipStream_t s) {
    ConvKParams K{a, (int)(a.d_inner + 2 * a.dstate), a.p_fixed == nullptr ? 1 : 0};
    const int64_t per_block = (kConvThreads / 64) * kConvTL;
    dim3 grid((unsigned)(K.ch / 64), (unsigned)((a.len + per_block - 1) / per_block),
              (unsigned)a.batch);
    conv_silu_kernel<<<grid, kConvThreads, 0, s>>>(K);
    fm_status st = check_launch("conv_silu_kernel");
    if (st != FM_OK || !K.dynamic) return st;
    const int64_t total = a.batch * a.len * K.ch;
    int g = (int)((total / 4 + kConvThreads - 1) / kConvThreads);
    if (g > 4096) g = 4096;
    if (g < 1) g = 1;
    requant_kernel<<<g, kConvThreads, 0, s>>>(K, total);
    return check_launch("requant_kernel");
}

}  // namespace fm
