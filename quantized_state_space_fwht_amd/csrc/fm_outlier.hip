// Baselines of the outlier study: per-tensor int8 quantization without the
// Hadamard rotation, and SmoothQuant-style per-channel smoothing (the
// comparison behind Fig. 3 and Table II of the FastMamba paper on the review
// page, and the outlier channels of the Mamba-PTQ abstract: a few activation
// channels with large values set a per-tensor scale that wastes the others).
//
//   per-tensor: c = 127 / max|x| (1 if the max is 0), q = sat8(rint(x * c)),
//               scale 1 / c — fm_hadamard_quant's arithmetic without H.
//   smoothing (alpha = 1/2): s_j = sqrt(max_i |x_ij|) / sqrt(max_n |w_nj|)
//               (1 if either max is 0); x' = x / s_j, w' = w * s_j column by
//               column, so x' w'^T = x w^T in exact arithmetic.
#include "fm_internal.hpp"

namespace fm {

constexpr int kOutThreads = 256;

// grid maximum of |x| over n4 float4 values (amax holds 0 on entry)
__global__ __launch_bounds__(kOutThreads) void absmax_kernel(const float4* __restrict__ x,
                                                             int64_t n4, float* amax) {
    float m = 0.0f;
    for (int64_t i = (int64_t)blockIdx.x * kOutThreads + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * kOutThreads)
        m = fmaxf(m, absmax4(x[i]));
    m = wave_max_f32(m);
    if ((threadIdx.x & 63) == 0 && m > 0.0f) atomic_max_nonneg_f32(amax, m);
}

__global__ __launch_bounds__(kOutThreads) void quant_per_tensor_kernel(
    const float4* __restrict__ x, int64_t n4, const float* amax, uint32_t* __restrict__ q,
    float* scale_out) {
    const float a = *amax;
    const float c = a == 0.0f ? 1.0f : 127.0f / a;
    if (blockIdx.x == 0 && threadIdx.x == 0) *scale_out = 1.0f / c;
    for (int64_t i = (int64_t)blockIdx.x * kOutThreads + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * kOutThreads)
        q[i] = quant_pack4(x[i], c);
}

// column maxima of |x| [rows, k]: thread per column, rows in order (coalesced
// across the wave); a grid of column blocks x row blocks, combined atomically
__global__ __launch_bounds__(kOutThreads) void col_absmax_kernel(const float* __restrict__ x,
                                                                 int64_t rows, int64_t k,
                                                                 int64_t rows_per_block,
                                                                 float* colmax) {
    const int64_t j = (int64_t)blockIdx.x * kOutThreads + threadIdx.x;
    if (j >= k) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < rows ? r0 + rows_per_block : rows;
    float m = 0.0f;
    for (int64_t r = r0; r < r1; ++r) m = fmaxf(m, fabsf(x[r * k + j]));
    if (m > 0.0f) atomic_max_nonneg_f32(&colmax[j], m);
}

__global__ __launch_bounds__(kOutThreads) void smooth_factor_kernel(const float* ax,
                                                                    const float* aw, int64_t k,
                                                                    float* s) {
    const int64_t j = (int64_t)blockIdx.x * kOutThreads + threadIdx.x;
    if (j >= k) return;
    const float a = ax[j], b = aw[j];
    s[j] = (a > 0.0f && b > 0.0f) ? sqrtf(a) / sqrtf(b) : 1.0f;
}

__global__ __launch_bounds__(kOutThreads) void scale_columns_kernel(
    const float* __restrict__ x, int64_t rows, int64_t k, const float* __restrict__ s, int divide,
    float* __restrict__ out) {
    const int64_t n = rows * k;
    for (int64_t i = (int64_t)blockIdx.x * kOutThreads + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kOutThreads) {
        const float sj = s[i % k];
        out[i] = divide ? x[i] / sj : x[i] * sj;
    }
}

static unsigned grid_for(int64_t n, int64_t cap = 4096) {
    int64_t g = (n + kOutThreads - 1) / kOutThreads;
    return (unsigned)(g < 1 ? 1 : (g > cap ? cap : g));
}

fm_status quant_per_tensor_run(const float* x, int64_t n, int8_t* q, float* scale_out,
                               float* amax_ws, hipStream_t s) {
    fm_status st;
    if ((st = zero_words(amax_ws, 1, s)) != FM_OK) return st;
    const int64_t n4 = n / 4;
    absmax_kernel<<<grid_for(n4, 1024), kOutThreads, 0, s>>>((const float4*)x, n4, amax_ws);
    if ((st = check_launch("absmax_kernel")) != FM_OK) return st;
    quant_per_tensor_kernel<<<grid_for(n4), kOutThreads, 0, s>>>((const float4*)x, n4, amax_ws,
                                                                 (uint32_t*)q, scale_out);
    return check_launch("quant_per_tensor_kernel");
}

fm_status smooth_scales_run(const float* x, int64_t rows, const float* w, int64_t n, int64_t k,
                            float* s_out, float* ws, hipStream_t s) {
    fm_status st;
    float* ax = ws;
    float* aw = ws + k;
    if ((st = zero_words(ws, 2 * k, s)) != FM_OK) return st;
    const unsigned gx = (unsigned)((k + kOutThreads - 1) / kOutThreads);
    auto colmax = [&](const float* src, int64_t r, float* dst) {
        const int64_t per = 256;  // rows per block
        const unsigned gy = (unsigned)((r + per - 1) / per);
        if (r > 0) col_absmax_kernel<<<dim3(gx, gy), kOutThreads, 0, s>>>(src, r, k, per, dst);
        return check_launch("col_absmax_kernel");
    };
    if ((st = colmax(x, rows, ax)) != FM_OK) return st;
    if ((st = colmax(w, n, aw)) != FM_OK) return st;
    smooth_factor_kernel<<<gx, kOutThreads, 0, s>>>(ax, aw, k, s_out);
    return check_launch("smooth_factor_kernel");
}

fm_status scale_columns_run(const float* x, int64_t rows, int64_t k, const float* sc, int divide,
                            float* out, hipStream_t s) {
    if (rows * k == 0) return FM_OK;
    scale_columns_kernel<<<grid_for(rows * k), kOutThreads, 0, s>>>(x, rows, k, sc, divide, out);
    return check_launch("scale_columns_kernel");
}

}  // namespace fm
