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
#include <type_traits>

#include "fm_internal.hpp"

namespace fm {

constexpr int kGateMaxD = 8192;
constexpr int kGateWaves = 4;     // many rows: a workgroup of 4 waves per row
constexpr int kGateStepWaves = 16;  // one-token step (few rows): 16 waves per row
// gate values per thread whose loads go out together: a round of 4 waves covers
// 2560 values, one of 16 waves 5120 (whole rounds at d_inner 5120 either way)
template <int W> constexpr int kGatePer = W == kGateStepWaves ? 5 : 10;

// One workgroup of W waves per row.  Phase 1: every thread computes gate
// values g_i (any split: each is independent) into LDS.  Phase 2: wave 0
// forms the sum of squares in the fixed order (lane l adds g_i^2 for
// i = l, l+64, ... ascending, then the xor tree).  Phase 3: the 256-blocks
// are normalized, rotated and quantized, block b by wave b % W.  With
// `rowmax` set (one-token step), the rotated row goes to rot_ws and its
// maximum to rowmax[row]; one pass over all rows then forms the codes with the
// tensor scale from those maxima.
template <int W>
__global__ __launch_bounds__(64 * W) void gate_norm_kernel(GateArgs G) {
    extern __shared__ __attribute__((aligned(16))) float row_buf[];  // d_inner floats
    __shared__ NauLds tab;
    __shared__ float rs_r;
    __shared__ float wmax[W];
    if (!G.sz) {  // SiLU(z) formed here
        nau_lds_init(tab);
        __syncthreads();
    }
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int64_t row = blockIdx.x;
    const int D = (int)G.d_inner;
    // one-token form (few rows, latency-bound): the norm weights of this wave's
    // first 256-block, loaded ahead of phase 1.  With many rows the workgroups
    // fill the wave slots and the longer-held registers cost more than this hides.
    constexpr bool kAhead = W == kGateStepWaves;
    float4 w_first = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (kAhead && wave < D / 256) w_first = reinterpret_cast<const float4*>(G.norm_w)[wave * 64 + lane];
    const float ysc = ldexpf(1.0f, -(G.p[1] + 8));
    const int32_t* yr = G.y + row * D;
    const float* zr = G.sz ? G.sz + row * D : G.z + row * G.z_stride;
    // phase 1: kGatePer elements per thread per round, loads of a round issued
    // together; rounds wholly inside the row (D is a multiple of 256, so a round
    // is whole for every thread or for none) run without per-element guards, and
    // whether SiLU(z) is formed here is decided once, so a round is straight-line
    // code whose independent SiLU chains interleave
    auto gate_round = [&](int i0, auto guarded, auto silu) __attribute__((always_inline)) {
        constexpr bool kG = decltype(guarded)::value, kSilu = decltype(silu)::value;
        int32_t yv[kGatePer<W>];
        float zv[kGatePer<W>];
#pragma unroll
        for (int k = 0; k < kGatePer<W>; ++k) {
            const int i = i0 + 64 * W * k;
            yv[k] = !kG || i < D ? yr[i] : 0;
            zv[k] = !kG || i < D ? zr[i] : 0.0f;
        }
#pragma unroll
        for (int k = 0; k < kGatePer<W>; ++k) {
            const int i = i0 + 64 * W * k;
            if (!kG || i < D) {
                const float yf = (float)yv[k] * ysc;
                float sz = zv[k];
                if constexpr (kSilu) sz = (float)nau_silu_d(f2d_sat(rintf(sz * 65536.0f)), tab) * 0x1p-16f;
                row_buf[i] = yf * sz;
            }
        }
    };
    constexpr int kRound = kGatePer<W> * 64 * W;
    auto phase1 = [&](auto silu) __attribute__((always_inline)) {
        int i0 = tid;
        for (; i0 - tid + kRound <= D; i0 += kRound) gate_round(i0, std::false_type{}, silu);
        if (i0 < D) gate_round(i0, std::true_type{}, silu);
    };
    if (G.sz) phase1(std::false_type{});
    else phase1(std::true_type{});
    __syncthreads();
    if (G.step_small && row == 0 && wave == W - 1) {
        // while wave 0 sums: the in_proj epilogue's slotted maxima into the call's
        // block (that kernel has completed; the out_proj product publishes it)
        const int32_t xbc = slots_wave_max(G.step_slots + kRegionXbc * kSlotRegionWords);
        int32_t pm[3];
#pragma unroll
        for (int i = 0; i < 3; ++i)
            pm[i] = slots_wave_max(G.step_slots + (kRegionConvX + i) * kSlotRegionWords);
        if (lane == 0) {
            G.step_small[kAmaxXbc] = (uint32_t)xbc;
#pragma unroll
            for (int i = 0; i < 3; ++i) G.step_small[kAmaxQ + i] = (uint32_t)pm[i];
        }
    }
    // phase 2: the fixed-order sum of squares
    if (wave == 0) {
        // ascending i within this lane (the fixed order): groups of 16 steps of
        // 64, then the rest in groups of 4 (D % 256 == 0), no per-element guards
        float a = 0.0f;
        int i0 = lane;
        for (; i0 - lane + 16 * 64 <= D; i0 += 16 * 64) {
            float g[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) g[k] = row_buf[i0 + 64 * k];
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const float g2 = g[k] * g[k];
                a = a + g2;
            }
        }
        for (; i0 < D; i0 += 4 * 64) {
            float g[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) g[k] = row_buf[i0 + 64 * k];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float g2 = g[k] * g[k];
                a = a + g2;
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
        const float4 w = kAhead && blk == wave ? w_first
                                                : *reinterpret_cast<const float4*>(&G.norm_w[base]);
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

}  // namespace fm
