// Narrow decode-state caches: conversion of an int32 state (as a prefill
// leaves it) to 16- or 24-bit codes on a power-of-two coarser grid and back,
// and the largest |state| for choosing the grid.  The state is read and
// written once per decoded token, so its width sets the decode step's memory
// traffic (FastMamba review, "What carries the argument": power-of-two scaling
// makes every SSM rescaling a shift).
//
// Codes: c = clamp(floor((h + 2^(shift-1)) / 2^shift), -2^(bits-1), 2^(bits-1)-1)
// (no rounding term at shift 0); stored as int16 or as the low 24 bits of
// the two's complement in three little-endian bytes.  These kernels run once
// per prefill, not per token: one element per thread, byte stores for the
// packed form.
#include "fm_internal.hpp"

namespace fm {

__global__ __launch_bounds__(256) void state_narrow_kernel(const int32_t* __restrict__ h, int64_t n,
                                                           int bits, int shift,
                                                           uint8_t* __restrict__ out) {
    const int32_t lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
    const int64_t half = ((int64_t)1 << shift) >> 1;
    const int nb = bits / 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t q = ((int64_t)h[i] + half) >> shift;
        const uint32_t c = (uint32_t)(int32_t)(q < lo ? lo : (q > hi ? hi : q));
        for (int k = 0; k < nb; ++k) out[i * nb + k] = (uint8_t)(c >> (8 * k));
    }
}

__global__ __launch_bounds__(256) void state_widen_kernel(const uint8_t* __restrict__ c, int64_t n,
                                                          int bits, int shift,
                                                          int32_t* __restrict__ out) {
    const int nb = bits / 8;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        uint32_t u = 0;
        for (int k = 0; k < nb; ++k) u |= (uint32_t)c[i * nb + k] << (8 * k);
        const int32_t v = (int32_t)(u << (32 - bits)) >> (32 - bits);  // sign-extend
        out[i] = v * (1 << shift);
    }
}

__global__ __launch_bounds__(256) void state_absmax_kernel(const int32_t* __restrict__ h, int64_t n,
                                                           uint32_t* __restrict__ amax) {
    uint32_t m = 0;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int32_t v = h[i];
        const uint32_t a = v < 0 ? 0u - (uint32_t)v : (uint32_t)v;  // |INT32_MIN| = 2^31
        m = a > m ? a : m;
    }
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)m, k, 64);
        m = o > m ? o : m;
    }
    __shared__ uint32_t wm[4];  // one atomic per workgroup: they all hit one word
    if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = wm[0];
        for (int k = 1; k < 4; ++k) m = wm[k] > m ? wm[k] : m;
        if (m) atomicMax(amax, m);
    }
}

static unsigned state_grid(int64_t n, int64_t cap = 4096) {
    const int64_t g = (n + 255) / 256;
    return (unsigned)(g < cap ? (g < 1 ? 1 : g) : cap);
}

fm_status state_narrow_run(const int32_t* h, int64_t n, int bits, int shift, void* out,
                           hipStream_t s) {
    if (n == 0) return FM_OK;
    state_narrow_kernel<<<state_grid(n), 256, 0, s>>>(h, n, bits, shift, (uint8_t*)out);
    return check_launch("state_narrow_kernel");
}

fm_status state_widen_run(const void* c, int64_t n, int bits, int shift, int32_t* out,
                          hipStream_t s) {
    if (n == 0) return FM_OK;
    state_widen_kernel<<<state_grid(n), 256, 0, s>>>((const uint8_t*)c, n, bits, shift, out);
    return check_launch("state_widen_kernel");
}

fm_status state_absmax_run(const int32_t* h, int64_t n, uint32_t* amax, hipStream_t s) {
    if (n == 0) return FM_OK;
    state_absmax_kernel<<<state_grid(n, 1024), 256, 0, s>>>(h, n, amax);
    return check_launch("state_absmax_kernel");
}

}  // namespace fm
