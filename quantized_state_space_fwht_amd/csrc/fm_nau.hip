// The nonlinear approximation unit as an elementwise call: e^x, SoftPlus and
// SiLU in Q.16 (review page of FastMamba, "What carries the argument": one
// 8-segment first-order approximation of 2^v serves e^x = 2^(x log2 e) and
// SoftPlus(x) = x + SoftPlus(-x); Eq. (5), Section III-B.2).
#include "fm_internal.hpp"

namespace fm {

// nine Q.30 knots of the 2^f unit, by value (use == 0: the chord table)
struct NauKnots {
    int64_t y[9];
    int use;
};

__global__ __launch_bounds__(256) void nau_eval_kernel(int fn, const int32_t* __restrict__ x,
                                                       int32_t* __restrict__ y, int64_t n,
                                                       NauKnots kn) {
    __shared__ NauLds tab;
    if (kn.use) {
        if (threadIdx.x < 8) nau_lds_set(tab, threadIdx.x, kn.y[threadIdx.x], kn.y[threadIdx.x + 1]);
    } else {
        nau_lds_init(tab);
    }
    __syncthreads();
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t v = x[i];
        int32_t r;
        if (fn == FM_NAU_EXP) r = nau_exp_f(v > 0 ? 0 : v, tab);
        else if (fn == FM_NAU_SOFTPLUS) r = nau_softplus_f(v, tab);
        else r = nau_silu_f(v, tab);
        y[i] = r;
    }
}

fm_status nau_run(int fn, const int32_t* x, int32_t* y, int64_t n, hipStream_t s,
                  const int64_t* knots) {
    if (n == 0) return FM_OK;
    int64_t g = (n + 255) / 256;
    if (g > 8192) g = 8192;
    NauKnots kn{};
    if (knots) {
        for (int i = 0; i < 9; ++i) kn.y[i] = knots[i];
        kn.use = 1;
    }
    nau_eval_kernel<<<(unsigned)g, 256, 0, s>>>(fn, x, y, n, kn);
    return check_launch("nau_eval_kernel");
}

}  // namespace fm
