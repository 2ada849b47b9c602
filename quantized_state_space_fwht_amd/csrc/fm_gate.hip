// Output gate y * SiLU(z), gated RMSNorm, then the Hadamard rotation and
// per-tensor int8 quantization of the out_proj input (Fig. 2 of the FastMamba
// paper: gate, RMSNorm and out_proj; the out_proj input is rotated and
// quantized like the in_proj input, "What carries the argument").
//
// One workgroup per row.  The sum of squares follows one fixed float32 order
// (lane l adds g_i^2 for i = l, l+64, ... ascending; then a[l] += a[l^k] for
// k = 32..1), because the normed values become int8 codes and a different
// rounding could flip one.  The row is staged in LDS and re-read in the
// 4-per-lane layout of the 256-point transform.
#include "fm_internal.hpp"

namespace fm {

__device__ __forceinline__ float4 fwht256_lane_g(float4 v, int lane) {
    float t0 = v.x + v.y, t1 = v.x - v.y, t2 = v.z + v.w, t3 = v.z - v.w;
    v.x = t0 + t2;
    v.z = t0 - t2;
    v.y = t1 + t3;
    v.w = t1 - t3;
    // stage m: the lane with bit m clear keeps a + b, its partner b' = a - b;
    // fma(+-1, v, p) rounds p + v / p - v exactly as the plain sums do
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

// sum of squares in the fixed order, identical in every lane
__device__ __forceinline__ float row_sumsq(float a) {
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) a = a + __shfl_xor(a, k, 64);
    return a;
}

constexpr int kGateMaxD = 8192;
constexpr int kGateWaves = 4;

// One workgroup of 4 waves per row.  Phase 1: every thread computes gate
// values g_i (any split: each is independent) into LDS.  Phase 2: wave 0
// forms the sum of squares in the fixed order (lane l adds g_i^2 for
// i = l, l+64, ... ascending, then the xor tree).  Phase 3: the 256-blocks
// are normalized, rotated and quantized, block b by wave b % 4.
__global__ __launch_bounds__(64 * kGateWaves) void gate_norm_kernel(GateArgs G) {
    extern __shared__ __attribute__((aligned(16))) float row_buf[];  // d_inner floats
    __shared__ NauLds tab;
    __shared__ float rs_r;
    __shared__ float wmax[kGateWaves];
    nau_lds_init(tab);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row = blockIdx.x;
    const int D = (int)G.d_inner;
    const float ysc = ldexpf(1.0f, -(G.p[1] + 8));
    const int32_t* yr = G.y + row * D;
    const float* zr = G.z + row * G.z_stride;
    // phase 1: four elements per thread per round, loads of a round issued together
    for (int i0 = tid; i0 < D; i0 += 4 * 64 * kGateWaves) {
        int32_t yv[4];
        float zv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + 64 * kGateWaves * k;
            yv[k] = i < D ? yr[i] : 0;
            zv[k] = i < D ? zr[i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + 64 * kGateWaves * k;
            const float yf = (float)yv[k] * ysc;
            const int32_t zq = f2i_sat(rintf(zv[k] * 65536.0f));
            const float sz = (float)nau_silu_f(zq, tab) * 0x1p-16f;
            if (i < D) row_buf[i] = yf * sz;
        }
    }
    __syncthreads();
    // phase 2: the fixed-order sum of squares
    if (wave == 0) {
        float a = 0.0f;
        for (int i = lane; i < D; i += 64) {
            const float g = row_buf[i];
            const float g2 = g * g;
            a = a + g2;  // ascending i within this lane: the fixed order
        }
        const float ss = row_sumsq(a);
        const float ms = ss / (float)D;
        if (lane == 0) rs_r = 1.0f / sqrtf(ms + 1e-5f);
    }
    __syncthreads();
    const float r = rs_r;
    float c = 0.0f;
    if (G.mode == FM_SCALE_STATIC) c = ldexpf((float)G.scoe, -G.sshift);
    float m = 0.0f;
    for (int blk = wave; blk < D / 256; blk += kGateWaves) {
        const int base = blk * 256 + lane * 4;
        float4 g = *reinterpret_cast<const float4*>(&row_buf[base]);
        const float4 w = *reinterpret_cast<const float4*>(&G.norm_w[base]);
        float4 n;
        n.x = (g.x * r) * w.x;
        n.y = (g.y * r) * w.y;
        n.z = (g.z * r) * w.z;
        n.w = (g.w * r) * w.w;
        if (G.normed_out) *reinterpret_cast<float4*>(&G.normed_out[row * D + base]) = n;
        const float4 v = fwht256_lane_g(n, lane);
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
        if (G.mode == FM_SCALE_DYNAMIC) {
            *reinterpret_cast<float4*>(&G.rot_ws[row * D + base]) = v;
        } else {
            char4 q;
            q.x = (signed char)fminf(fmaxf(rintf(v.x * c), -127.0f), 127.0f);
            q.y = (signed char)fminf(fmaxf(rintf(v.y * c), -127.0f), 127.0f);
            q.z = (signed char)fminf(fmaxf(rintf(v.z * c), -127.0f), 127.0f);
            q.w = (signed char)fminf(fmaxf(rintf(v.w * c), -127.0f), 127.0f);
            *reinterpret_cast<char4*>(&G.q[row * D + base]) = q;
        }
    }
    m = wave_max_f32(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    if (tid == 0) {
        m = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
        if (G.mode == FM_SCALE_DYNAMIC) atomic_max_nonneg_f32(G.amax_ws, m);
        if (G.amax_stats) atomic_max_nonneg_f32(G.amax_stats, m);
        if (G.mode == FM_SCALE_STATIC && row == 0) *G.scale_out = 1.0f / c;
    }
}

fm_status gate_run(const GateArgs& g, hipStream_t s) {
    if (g.d_inner > kGateMaxD)
        return fail(FM_ERR_SHAPE, "gate: d_inner %lld > %d", (long long)g.d_inner, kGateMaxD);
    if (g.rows > 0) {
        gate_norm_kernel<<<(unsigned)g.rows, 64 * kGateWaves, (size_t)g.d_inner * sizeof(float),
                           s>>>(g);
        fm_status st = check_launch("gate_norm_kernel");
        if (st != FM_OK) return st;
    }
    if (g.mode == FM_SCALE_DYNAMIC)
        return hq_quant_rotated(g.rot_ws, g.rows, g.d_inner, FM_SCALE_DYNAMIC, 0, 0, g.amax_ws, g.q,
                                g.scale_out, s);
    if (g.rows == 0) return hq_quant_rotated(g.rot_ws, 0, g.d_inner, g.mode, g.scoe, g.sshift,
                                             nullptr, g.q, g.scale_out, s);
    return FM_OK;
}

// RMSNorm of the residual stream with unit weight (pre-norm stacks): one
// workgroup of 4 waves per row; the row is staged in LDS by all waves, wave 0
// forms the fixed-order sum of squares, all waves write the normed row.
__global__ __launch_bounds__(64 * kGateWaves) void rmsnorm_rows_kernel(
    const float* __restrict__ h, int d, float* __restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) float hrow[];  // d floats
    __shared__ float rs_r;
    const int tid = threadIdx.x, lane = tid & 63;
    const int64_t row = blockIdx.x;
    const float* hr = h + row * d;
    for (int i = tid; i < d; i += 64 * kGateWaves) hrow[i] = hr[i];
    __syncthreads();
    if (tid < 64) {
        float a = 0.0f;
        for (int i = lane; i < d; i += 64) {
            const float v = hrow[i];
            const float v2 = v * v;
            a = a + v2;
        }
        const float ss = row_sumsq(a);
        if (lane == 0) rs_r = 1.0f / sqrtf(ss / (float)d + 1e-5f);
    }
    __syncthreads();
    const float r = rs_r;
    for (int i = tid; i < d; i += 64 * kGateWaves) out[row * d + i] = (hrow[i] * r) * 1.0f;
}

fm_status rmsnorm_rows_run(const float* h, int64_t rows, int64_t d, float* out, hipStream_t s) {
    if (rows == 0) return FM_OK;
    rmsnorm_rows_kernel<<<(unsigned)rows, 64 * kGateWaves, (size_t)d * sizeof(float), s>>>(
        h, (int)d, out);
    return check_launch("rmsnorm_rows_kernel");
}

}  // namespace fm
