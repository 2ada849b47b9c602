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

constexpr int kGateMaxD = 8192;
constexpr int kGateWaves = 4;     // many rows: a workgroup of 4 waves per row
constexpr int kGateStepWaves = 16;  // one-token step (few rows): 16 waves per row
constexpr int kGatePer = 8;       // gate values per thread whose loads go out together

// One workgroup of W waves per row.  Phase 1: every thread computes gate
// values g_i (any split: each is independent) into LDS.  Phase 2: wave 0
// forms the sum of squares in the fixed order (lane l adds g_i^2 for
// i = l, l+64, ... ascending, then the xor tree).  Phase 3: the 256-blocks
// are normalized, rotated and quantized, block b by wave b % W.  With
// `rowmax` set (one-token step), the rotated row goes to rot_ws and its
// maximum to rowmax[row]; the out_proj product quantizes.
template <int W>
__global__ __launch_bounds__(64 * W) void gate_norm_kernel(GateArgs G) {
    extern __shared__ __attribute__((aligned(16))) float row_buf[];  // d_inner floats
    __shared__ NauLds tab;
    __shared__ float rs_r;
    __shared__ float wmax[W];
    nau_lds_init(tab);
    __syncthreads();
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row = blockIdx.x;
    const int D = (int)G.d_inner;
    const float ysc = ldexpf(1.0f, -(G.p[1] + 8));
    const int32_t* yr = G.y + row * D;
    const float* zr = G.sz ? G.sz + row * D : G.z + row * G.z_stride;
    // phase 1: kGatePer elements per thread per round, loads of a round issued together
    for (int i0 = tid; i0 < D; i0 += kGatePer * 64 * W) {
        int32_t yv[kGatePer];
        float zv[kGatePer];
#pragma unroll
        for (int k = 0; k < kGatePer; ++k) {
            const int i = i0 + 64 * W * k;
            yv[k] = i < D ? yr[i] : 0;
            zv[k] = i < D ? zr[i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kGatePer; ++k) {
            const int i = i0 + 64 * W * k;
            if (i < D) {
                const float yf = (float)yv[k] * ysc;
                float sz = zv[k];
                if (!G.sz) sz = (float)nau_silu_f(f2i_sat(rintf(sz * 65536.0f)), tab) * 0x1p-16f;
                row_buf[i] = yf * sz;
            }
        }
    }
    __syncthreads();
    // phase 2: the fixed-order sum of squares
    if (wave == 0) {
        float a = 0.0f;
        for (int i0 = lane; i0 < D; i0 += 16 * 64) {  // D % 256 == 0: 4 steps at least
            float g[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) g[k] = i0 + 64 * k < D ? row_buf[i0 + 64 * k] : 0.0f;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                if (i0 + 64 * k < D) {
                    const float g2 = g[k] * g[k];
                    a = a + g2;  // ascending i within this lane: the fixed order
                }
            }
        }
        const float ss = wave_sum_fixed(a);
        const float ms = ss / (float)D;
        if (lane == 0) rs_r = 1.0f / sqrtf(ms + 1e-5f);
    }
    __syncthreads();
    const float r = rs_r;
    const bool dyn = G.mode == FM_SCALE_DYNAMIC;
    float c = 0.0f;
    if (!dyn) c = ldexpf((float)G.scoe, -G.sshift);
    float m = 0.0f;
    QStat st;
    for (int blk = wave; blk < D / 256; blk += W) {
        const int base = blk * 256 + lane * 4;
        float4 g = *reinterpret_cast<const float4*>(&row_buf[base]);
        const float4 w = *reinterpret_cast<const float4*>(&G.norm_w[base]);
        float4 n;
        n.x = (g.x * r) * w.x;
        n.y = (g.y * r) * w.y;
        n.z = (g.z * r) * w.z;
        n.w = (g.w * r) * w.w;
        if (G.normed_out) *reinterpret_cast<float4*>(&G.normed_out[row * D + base]) = n;
        const float4 v = fwht256_lane(n, lane);
        m = fmaxf(m, absmax4(v));
        if (dyn || G.rowmax) {
            *reinterpret_cast<float4*>(&G.rot_ws[row * D + base]) = v;
        } else {
            *reinterpret_cast<char4*>(&G.q[row * D + base]) = quant4(v, c);
            if (G.qs) quant_stat4(st, v, c, 1.0f / c);
        }
    }
    if (G.qs && !dyn && !G.rowmax) qstat_flush(st, G.qs, FM_QP_G);
    m = wave_max_f32(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    if (tid == 0) {
        m = wmax[0];
        for (int k = 1; k < W; ++k) m = fmaxf(m, wmax[k]);
        if (G.rowmax) {
            G.rowmax[row] = m;
            return;
        }
        if (dyn) slot_max(G.amax_slots, row, (int32_t)__float_as_uint(m));
        if (G.amax_stats) atomic_max_nonneg_f32(G.amax_stats, m);
        if (!dyn && row == 0) *G.scale_out = 1.0f / c;
    }
}

fm_status gate_run(const GateArgs& g, hipStream_t s) {
    if (g.d_inner > kGateMaxD)
        return fail(FM_ERR_SHAPE, "gate: d_inner %lld > %d", (long long)g.d_inner, kGateMaxD);
    const size_t lds = (size_t)g.d_inner * sizeof(float);
    if (g.rowmax) {  // one-token step: rotated rows and row maxima only
        if (g.rows > 0)
            gate_norm_kernel<kGateStepWaves><<<(unsigned)g.rows, 64 * kGateStepWaves, lds, s>>>(g);
        return check_launch("gate_norm_kernel");
    }
    if (g.rows > 0) {
        gate_norm_kernel<kGateWaves><<<(unsigned)g.rows, 64 * kGateWaves, lds, s>>>(g);
        fm_status st = check_launch("gate_norm_kernel");
        if (st != FM_OK) return st;
    }
    if (g.mode == FM_SCALE_DYNAMIC)
        return hq_quant_rotated(g.rot_ws, g.rows, g.d_inner, FM_SCALE_DYNAMIC, 0, 0, g.amax_ws,
                                g.amax_slots, g.q, g.scale_out, s, g.qs, FM_QP_G);
    if (g.rows == 0) return hq_quant_rotated(g.rot_ws, 0, g.d_inner, g.mode, g.scoe, g.sshift,
                                             nullptr, nullptr, g.q, g.scale_out, s);
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
        const float ss = wave_sum_fixed(a);
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
