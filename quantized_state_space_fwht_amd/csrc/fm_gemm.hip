// W8A8 GEMM on gfx950 int8 matrix cores: C = A * B^T, int32 accumulation,
// float dequantization epilogue (review page abstract: 8-bit linear layers;
// "What carries the argument": Y = (XH)(H^T W^T)).
//
// Tile 128 x 128 x 64 per workgroup of 4 waves (2 x 2), each wave 64 x 64 as
// 4 x 4 v_mfma_i32_16x16x64_i8 tiles.  A and B tiles are staged through LDS
// (double-buffered, rows padded to 80 bytes so the 16-byte fragment reads
// hit distinct banks).  For the MFMA, lane l supplies row (l % 16) and the
// 16 k-values [16*(l/16), 16*(l/16)+16) of its 64-wide k slice, for A and B
// alike, so every k pairs with itself whatever byte order the instruction
// uses inside a lane.  Result lane l holds rows 4*(l/16)+i, column l % 16.
#include "fm_internal.hpp"

namespace fm {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLdsRow = kBK + 16;  // bytes per staged row (padding against bank conflicts)
constexpr int kGemmThreads = 256;

struct GemmParams {
    const int8_t* a;
    const int8_t* b;
    int64_t m, n, k;
    GemmEpilogue ep;
};

__global__ __launch_bounds__(kGemmThreads) void gemm_i8_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(16))) int8_t As[2][kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][kBN * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.y * kBM;
    const int64_t n0 = (int64_t)blockIdx.x * kBN;
    const int64_t K = P.k;

    // global -> register staging: each thread moves 2 x 16 bytes of A and of B
    const int ld_row = tid >> 2;          // 0..63 (+64 for the second half)
    const int ld_col = (tid & 3) * 16;    // byte offset inside the 64-wide k slice
    int64_t ra0 = m0 + ld_row, ra1 = m0 + ld_row + 64;
    int64_t rb0 = n0 + ld_row, rb1 = n0 + ld_row + 64;
    // rows past the edge read the last valid row; their results are never stored
    ra0 = ra0 < P.m ? ra0 : P.m - 1;
    ra1 = ra1 < P.m ? ra1 : P.m - 1;
    rb0 = rb0 < P.n ? rb0 : P.n - 1;
    rb1 = rb1 < P.n ? rb1 : P.n - 1;
    const int8_t* pa0 = P.a + ra0 * K + ld_col;
    const int8_t* pa1 = P.a + ra1 * K + ld_col;
    const int8_t* pb0 = P.b + rb0 * K + ld_col;
    const int8_t* pb1 = P.b + rb1 * K + ld_col;

    v4i ga0, ga1, gb0, gb1;
    auto gload = [&](int64_t k0) {
        ga0 = *reinterpret_cast<const v4i*>(pa0 + k0);
        ga1 = *reinterpret_cast<const v4i*>(pa1 + k0);
        gb0 = *reinterpret_cast<const v4i*>(pb0 + k0);
        gb1 = *reinterpret_cast<const v4i*>(pb1 + k0);
    };
    auto lstore = [&](int buf) {
        *reinterpret_cast<v4i*>(&As[buf][ld_row * kLdsRow + ld_col]) = ga0;
        *reinterpret_cast<v4i*>(&As[buf][(ld_row + 64) * kLdsRow + ld_col]) = ga1;
        *reinterpret_cast<v4i*>(&Bs[buf][ld_row * kLdsRow + ld_col]) = gb0;
        *reinterpret_cast<v4i*>(&Bs[buf][(ld_row + 64) * kLdsRow + ld_col]) = gb1;
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int64_t KT = K / kBK;
    if (P.m > 0 && P.n > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();
    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * 16;
    int buf = 0;
    for (int64_t kt = 0; kt < KT; ++kt) {
        const bool more = kt + 1 < KT;
        if (more) gload((kt + 1) * kBK);
        v4i af[4], bf[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = *reinterpret_cast<const v4i*>(
                &As[buf][(wm * 64 + i * 16 + frag_row) * kLdsRow + frag_k]);
            bf[i] = *reinterpret_cast<const v4i*>(
                &Bs[buf][(wn * 64 + i * 16 + frag_row) * kLdsRow + frag_k]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        if (more) lstore(buf ^ 1);
        __syncthreads();
        buf ^= 1;
    }

    // epilogue
    const GemmEpilogue& ep = P.ep;
    float sab = 0.0f;
    if (ep.out) sab = (*ep.s_a) * (*ep.s_b);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = n0 + wn * 64 + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + r;
                if (row < P.m && col < P.n) {
                    int32_t v = acc[i][j][r];
                    if (ep.acc) ep.acc[row * ep.ld_acc + col] = v;
                    if (ep.out) {
                        float o = (float)v * sab;
                        if (ep.resid) o = ep.resid[row * ep.ld_resid + col] + o;
                        ep.out[row * ep.ld_out + col] = o;
                        if (col >= ep.amax_c0 && col < ep.amax_c1) amax = fmaxf(amax, fabsf(o));
                    }
                }
            }
        }
    }
    if (ep.amax) {
        amax = wave_max_f32(amax);
        if (lane == 0 && amax > 0.0f) atomic_max_nonneg_f32(ep.amax, amax);
    }
}

// ---------------------------------------------------------------- few rows (decode)
// M <= 64: weight traffic is the whole cost, so every workgroup streams its own
// 16 columns of B over the full K exactly once.  The 4 waves split K in four;
// each wave keeps MT (= ceil(M/16)) 16 x 16 accumulator tiles, and the
// partial tiles are added through LDS before the same epilogue as above.
constexpr int kSkU = 4;  // k-slices of 64 whose loads are issued together

template <int MT>
__global__ __launch_bounds__(kGemmThreads) void gemm_i8_few_rows_kernel(GemmParams P) {
    __shared__ __attribute__((aligned(16))) int32_t part[4][MT][64][4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * 16;
    const int64_t K = P.k, kq = K / 4;  // k range of this wave: [wave*kq, wave*kq + kq)
    const int frag_row = lane & 15, frag_k = (lane >> 4) * 16;
    int64_t rb = n0 + frag_row;
    rb = rb < P.n ? rb : P.n - 1;  // columns past the edge: computed, never stored
    const int8_t* pb = P.b + rb * K + wave * kq + frag_k;
    const int8_t* pa[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        int64_t ra = t * 16 + frag_row;
        ra = ra < P.m ? ra : P.m - 1;
        pa[t] = P.a + ra * K + wave * kq + frag_k;
    }
    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};
    const int64_t steps = kq / kBK;
    int64_t s0 = 0;
    for (; s0 + kSkU <= steps; s0 += kSkU) {
        v4i bf[kSkU], af[kSkU][MT];
#pragma unroll
        for (int u = 0; u < kSkU; ++u) {
            bf[u] = *reinterpret_cast<const v4i*>(pb + (s0 + u) * kBK);
#pragma unroll
            for (int t = 0; t < MT; ++t)
                af[u][t] = *reinterpret_cast<const v4i*>(pa[t] + (s0 + u) * kBK);
        }
#pragma unroll
        for (int u = 0; u < kSkU; ++u)
#pragma unroll
            for (int t = 0; t < MT; ++t)
                acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[u][t], bf[u], acc[t], 0, 0, 0);
    }
    for (; s0 < steps; ++s0) {
        const v4i bf = *reinterpret_cast<const v4i*>(pb + s0 * kBK);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const v4i af = *reinterpret_cast<const v4i*>(pa[t] + s0 * kBK);
            acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[t], 0, 0, 0);
        }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) *reinterpret_cast<v4i*>(&part[wave][t][lane][0]) = acc[t];
    __syncthreads();
    if (wave != 0) return;
    const GemmEpilogue& ep = P.ep;
    float sab = 0.0f;
    if (ep.out) sab = (*ep.s_a) * (*ep.s_b);
    float amax = 0.0f;
    const int64_t col = n0 + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t row = t * 16 + (lane >> 4) * 4 + r;
            // int32 sum of the four k quarters (exact: |acc| < 2^31 for any order)
            const int32_t v = part[0][t][lane][r] + part[1][t][lane][r] + part[2][t][lane][r] +
                              part[3][t][lane][r];
            if (row < P.m && col < P.n) {
                if (ep.acc) ep.acc[row * ep.ld_acc + col] = v;
                if (ep.out) {
                    float o = (float)v * sab;
                    if (ep.resid) o = ep.resid[row * ep.ld_resid + col] + o;
                    ep.out[row * ep.ld_out + col] = o;
                    if (col >= ep.amax_c0 && col < ep.amax_c1) amax = fmaxf(amax, fabsf(o));
                }
            }
        }
    }
    if (ep.amax) {
        amax = wave_max_f32(amax);
        if (lane == 0 && amax > 0.0f) atomic_max_nonneg_f32(ep.amax, amax);
    }
}

fm_status gemm_run(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k,
                   const GemmEpilogue& ep, hipStream_t s) {
    if (m == 0 || n == 0) return FM_OK;
    GemmParams P{a, b, m, n, k, ep};
    if (m <= 64 && k % (4 * kBK) == 0) {
        const unsigned g = (unsigned)((n + 15) / 16);
        switch ((m + 15) / 16) {
            case 1: gemm_i8_few_rows_kernel<1><<<g, kGemmThreads, 0, s>>>(P); break;
            case 2: gemm_i8_few_rows_kernel<2><<<g, kGemmThreads, 0, s>>>(P); break;
            case 3: gemm_i8_few_rows_kernel<3><<<g, kGemmThreads, 0, s>>>(P); break;
            default: gemm_i8_few_rows_kernel<4><<<g, kGemmThreads, 0, s>>>(P); break;
        }
        return check_launch("gemm_i8_few_rows_kernel");
    }
    dim3 grid((unsigned)((n + kBN - 1) / kBN), (unsigned)((m + kBM - 1) / kBM));
    gemm_i8_kernel<<<grid, kGemmThreads, 0, s>>>(P);
    return check_launch("gemm_i8_kernel");
}

}  // namespace fm
