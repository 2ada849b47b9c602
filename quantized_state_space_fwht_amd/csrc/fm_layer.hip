// The quantized Mamba2 mixer layer (Fig. 2 flow of the FastMamba paper:
// in_proj -> conv1d + SiLU -> SSM -> gated RMSNorm -> out_proj) assembled from
// the step kernels, plus the offline parameter preparation.
//
// Every step runs on the device; the dynamic scales and exponents flow from
// kernel to kernel through a small block at the head of the workspace and
// are never copied to the host.
#include "fm_internal.hpp"

namespace fm {

struct LayerWs {
    uint32_t* small;
    int32_t* slots;  // kRegions slot regions (grid maxima of the prefill passes)
    float* un;       // pre-norm output [T, dm]
    int8_t* u_q;     // [T, dm]
    float* v;        // [T, dip]
    int8_t* xbc_q;   // [T, ch]
    int32_t* s16;    // [T, ch]
    int8_t* x_q;     // [T, di]
    int8_t* b_q;     // [T, N]
    int8_t* c_q;     // [T, N]
    int32_t* y;      // [T, di]
    float* rot;      // [T, di]
    float* normed;   // [T, di]
    int8_t* g_q;     // [T, di]
    int32_t* dt;     // [T, H]
    int32_t* da;     // [T, H]
    void* scan_ws;   // scan prologue scalars
    float* rowmax;   // one-token step: [2, 64] row maxima (in_proj input, out_proj input)
    float* sz;       // one-token step: [T, di] SiLU(z) from the in_proj epilogue
    float* rs;       // stacks: [T] 1/rms of the pre-norm, from the dynamic maximum pass
    size_t bytes;
};

static LayerWs layer_ws(const fm_layer_desc* d, int64_t batch, int64_t len, void* base) {
    const int64_t T = batch * len;
    const int64_t dm = d->d_model, di = d->d_inner, N = d->dstate, H = d->nheads;
    const int64_t ch = di + 2 * N, dip = 2 * di + 2 * N + H;
    Arena ar(base);
    LayerWs w;
    w.small = ar.take<uint32_t>(kSmallWords);
    w.slots = ar.take<int32_t>((size_t)kRegions * kSlotRegionWords);
    w.un = ar.take<float>((size_t)T * dm);
    w.u_q = ar.take<int8_t>((size_t)T * dm);
    w.v = ar.take<float>((size_t)T * dip);
    w.xbc_q = ar.take<int8_t>((size_t)T * ch);
    w.s16 = ar.take<int32_t>((size_t)T * ch);
    w.x_q = ar.take<int8_t>((size_t)T * di);
    w.b_q = ar.take<int8_t>((size_t)T * N);
    w.c_q = ar.take<int8_t>((size_t)T * N);
    w.y = ar.take<int32_t>((size_t)T * di);
    w.rot = ar.take<float>((size_t)T * di);
    w.normed = ar.take<float>((size_t)T * di);
    w.g_q = ar.take<int8_t>((size_t)T * di);
    w.dt = ar.take<int32_t>((size_t)T * H);
    w.da = ar.take<int32_t>((size_t)T * H);
    w.scan_ws = ar.take<char>(scan_ws_bytes(batch, len, d->dstate));
    w.rowmax = ar.take<float>(T <= 64 ? 128 : 0);
    w.sz = ar.take<float>(T <= 64 ? (size_t)T * di : 0);
    w.rs = ar.take<float>((size_t)T);
    w.bytes = ar.used;
    return w;
}

size_t layer_ws_bytes(const fm_layer_desc* d, int64_t batch, int64_t len) {
    return layer_ws(d, batch, len, nullptr).bytes;
}

void layer_taps(const fm_layer_desc* d, int64_t batch, int64_t len, fm_layer_taps* t) {
    LayerWs w = layer_ws(d, batch, len, nullptr);
    auto off = [](const void* p) { return (size_t)(uintptr_t)p; };
    t->u_q = off(w.u_q);
    t->v = off(w.v);
    t->xbc_q = off(w.xbc_q);
    t->x_q = off(w.x_q);
    t->b_q = off(w.b_q);
    t->c_q = off(w.c_q);
    t->y = off(w.y);
    t->g_q = off(w.g_q);
    t->normed = off(w.normed);
    t->dt = off(w.dt);
    t->da = off(w.da);
}

// zero the small block and the slots of the slot regions; optionally load the
// exponents (static values or a device copy)
__global__ void layer_setup_kernel(uint32_t* small, int32_t* slots, const int32_t* p_src, int p0,
                                   int p1, int p2, int p3, int how) {
    const int i = threadIdx.x;
    for (int k = i; k < kSmallWords; k += blockDim.x) small[k] = 0u;
    for (int k = i; k < kRegions * kSlots; k += blockDim.x)
        slots[(k / kSlots) * kSlotRegionWords + (k % kSlots) * kSlotStride] = 0;
    __syncthreads();
    if (i == 0 && how != 0) {
        int32_t* p = (int32_t*)(small + kP);
        if (how == 1) {
            p[0] = p0;
            p[1] = p1;
            p[2] = p2;
            p[3] = p3;
        } else {
            for (int k = 0; k < 4; ++k) p[k] = p_src[k];
        }
    }
}

// ---------------------------------------------------------------- one-token step input
// A decode step has few rows (T = batch <= 64).  One workgroup per row stages
// the row in LDS, forms the pre-norm (wave 0: the fixed-order sum of squares as
// in norm_hq_kernel), rotates the 256-blocks and stores the rotated row
// and its maximum; the in_proj product turns them into codes with the tensor
// scale.  Workgroup 0 also zeroes the call's small block and the slot regions
// of the in_proj epilogue's maxima and loads the frozen exponents (nothing in
// this kernel reads them).
constexpr int kStepRowThreads = 256;
static_assert(kSmallWords <= kStepRowThreads, "workgroup 0 zeroes the small block in one pass");

struct StepRowsArgs {
    const float* u;
    int dm;
    int prenorm;
    const int32_t* p_src;  // frozen exponents [4]
    uint32_t* small;
    int32_t* slots;        // the layer's slot regions
    float* rot;            // [rows, dm]
    float* rowmax;         // [rows]
};

__global__ __launch_bounds__(kStepRowThreads) void step_rows_kernel(StepRowsArgs A) {
    extern __shared__ __attribute__((aligned(16))) float row[];  // dm floats
    __shared__ float rs_s;
    __shared__ float wmax[kStepRowThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    if (blockIdx.x == 0) {
        if (tid < kSmallWords)
            A.small[tid] = (tid >= kP && tid < kP + 4) ? (uint32_t)A.p_src[tid - kP] : 0u;
        // slots of max |SiLU| of x, B, C (three regions) and of max |xBC|
        if (tid < 4 * kSlots) {
            const int reg = tid / kSlots < 3 ? kRegionConvX + tid / kSlots : kRegionXbc;
            A.slots[reg * kSlotRegionWords + (tid % kSlots) * kSlotStride] = 0;
        }
    }
    const int dm = A.dm;
    const int64_t r = blockIdx.x;
    const float* ur = A.u + r * dm;
    for (int i0 = tid * 4; i0 < dm; i0 += 4 * 4 * kStepRowThreads) {  // 4 loads in flight
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + k * 4 * kStepRowThreads;
            v[k] = i < dm ? *reinterpret_cast<const float4*>(ur + i) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = i0 + k * 4 * kStepRowThreads;
            if (i < dm) *reinterpret_cast<float4*>(row + i) = v[k];
        }
    }
    __syncthreads();
    float rs = 1.0f;
    if (A.prenorm) {
        if (wave == 0) {
            // ascending i within this lane (the fixed order): groups of 16 steps of
            // 64, then the rest in groups of 4 (dm % 256 == 0), no per-element guards
            float a = 0.0f;
            int i0 = lane;
            for (; i0 - lane + 16 * 64 <= dm; i0 += 16 * 64) {
                float v[16];
#pragma unroll
                for (int k = 0; k < 16; ++k) v[k] = row[i0 + 64 * k];
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const float v2 = v[k] * v[k];
                    a = a + v2;
                }
            }
            for (; i0 < dm; i0 += 4 * 64) {
                float v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) v[k] = row[i0 + 64 * k];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float v2 = v[k] * v[k];
                    a = a + v2;
                }
            }
            const float ss = wave_sum_fixed(a);
            if (lane == 0) rs_s = 1.0f / sqrtf(ss / (float)dm + 1e-5f);
        }
        __syncthreads();
        rs = rs_s;
    }
    float m = 0.0f;
    for (int blk = wave; blk < dm / 256; blk += kStepRowThreads / 64) {
        float4 v = *reinterpret_cast<const float4*>(row + blk * 256 + lane * 4);
        if (A.prenorm) {
            v.x = (v.x * rs) * 1.0f;
            v.y = (v.y * rs) * 1.0f;
            v.z = (v.z * rs) * 1.0f;
            v.w = (v.w * rs) * 1.0f;
        }
        v = fwht256_lane(v, lane);
        m = fmaxf(m, absmax4(v));
        reinterpret_cast<float4*>(A.rot + r * dm + blk * 256)[lane] = v;
    }
    m = wave_max_f32(m);
    if (lane == 0) wmax[wave] = m;
    __syncthreads();
    if (tid == 0) {
        for (int k = 1; k < kStepRowThreads / 64; ++k) m = fmaxf(m, wmax[k]);
        A.rowmax[r] = fmaxf(m, wmax[0]);
    }
}

// Shared body of prefill (len tokens, fresh state) and decode (len = 1, cache).
fm_status layer_run(const fm_layer_desc* d, const fm_layer_weights* W, const fm_static_params* sp,
                    const float* u, int64_t batch, int64_t len, float* out, const fm_cache* cache,
                    fm_qparams* qp, void* workspace, bool decode, hipStream_t s,
                    const LayerOpts& opts, int state_bits, int state_shift, void* ssd_ws) {
    const int64_t T = batch * len;
    const int64_t dm = d->d_model, di = d->d_inner, N = d->dstate, H = d->nheads, P = d->headdim;
    const int64_t ch = di + 2 * N, dip = 2 * di + 2 * N + H;
    const fm_scale_mode mode = (fm_scale_mode)d->mode;
    const bool stat = mode == FM_SCALE_STATIC;
    LayerWs w = layer_ws(d, batch, len, workspace);
    fm_quant_stats* const qs = decode ? nullptr : opts.qs;  // prefill calls collect
    const bool keep = opts.keep;
    fm_status st;
    float* small_f = (float*)w.small;
    int32_t* small_i = (int32_t*)w.small;
    int32_t* pdev = small_i + kP;
    auto mark = [&](int i) -> fm_status {
        if (opts.ev[i] && hipEventRecord(opts.ev[i], s) != hipSuccess)
            return fail(FM_ERR_HIP, "hipEventRecord(stage event %d) failed", i);
        return FM_OK;
    };
    if ((st = mark(0)) != FM_OK) return st;

    // A decode step with few rows takes the fused form, six kernels: rotated
    // input rows; in_proj quantizing them on load, with the conv step in its
    // epilogue; the scan step; rotated gate rows; their codes (one pass);
    // out_proj, adding the residual and publishing the call's scalars.
    const bool step = decode && T <= 64;
    if (step) {
        StepRowsArgs a{};
        a.u = u;
        a.dm = (int)dm;
        a.prenorm = d->prenorm_residual ? 1 : 0;
        a.p_src = cache->p;
        a.small = w.small;
        a.slots = w.slots;
        a.rot = w.un;
        a.rowmax = w.rowmax;
        step_rows_kernel<<<(unsigned)T, kStepRowThreads, (size_t)dm * sizeof(float), s>>>(a);
        if ((st = check_launch("step_rows_kernel")) != FM_OK) return st;
    } else {
        // 0. setup: zero the per-call block, load exponents (static values or the cache's)
        if (decode)
            layer_setup_kernel<<<1, 64, 0, s>>>(w.small, w.slots, cache->p, 0, 0, 0, 0, 2);
        else if (stat)
            layer_setup_kernel<<<1, 64, 0, s>>>(w.small, w.slots, nullptr, sp->p[0], sp->p[1],
                                                sp->p[2], sp->p[3], 1);
        else
            layer_setup_kernel<<<1, 64, 0, s>>>(w.small, w.slots, nullptr, 0, 0, 0, 0, 0);
        if ((st = check_launch("layer_setup_kernel")) != FM_OK) return st;

        // 1-2. rotate + quantize the in_proj input (stacks: of the residual stream's
        // pre-norm, formed on the fly)
        if (d->prenorm_residual) {
            if ((st = norm_hq_run(u, T, dm, mode, stat ? sp->scoe[0] : 0, stat ? sp->sshift[0] : 0,
                                  w.u_q, small_f + kScaleU, stat ? small_f + kAmaxU : nullptr,
                                  small_f + kAmaxU, w.slots + kRegionU * kSlotRegionWords, w.rs,
                                  s, qs, FM_QP_U)) != FM_OK)
                return st;
        } else if ((st = hq_run(u, T, dm, mode, stat ? sp->scoe[0] : 0,
                                stat ? sp->sshift[0] : 0, w.u_q, small_f + kScaleU,
                                stat ? small_f + kAmaxU : nullptr, small_f + kAmaxU,
                                w.slots + kRegionU * kSlotRegionWords, s, qs, FM_QP_U)) != FM_OK) {
            return st;
        }
    }
    if ((st = mark(1)) != FM_OK) return st;
    // 3. in_proj W8A8, dequant, max |xBC| for the conv exponent
    {
        GemmEpilogue ep;
        ep.out = w.v;
        ep.ld_out = dip;
        ep.s_a = small_f + kScaleU;
        ep.s_b = W->s_w_in;
        // the conv pass reduces max |xBC| from a slot region when its exponents are
        // dynamic; the fused step and fixed exponents keep the one word
        if (step || !(stat || decode)) ep.amax_slots = w.slots + kRegionXbc * kSlotRegionWords;
        else ep.amax = small_f + kAmaxXbc;
        ep.amax_c0 = di;
        ep.amax_c1 = di + ch;
        if (step) {  // 2 fused: codes of the rotated rows with the tensor scale
            ep.a_f = w.un;
            ep.a_rowmax = w.rowmax;
            ep.a_mode = mode;
            ep.a_scoe = stat ? sp->scoe[0] : 0;
            ep.a_sshift = stat ? sp->sshift[0] : 0;
            ep.a_amax_out = small_f + kAmaxU;
            ep.a_scale_out = small_f + kScaleU;
            ep.a_q_tap = keep ? w.u_q : nullptr;
        }
        if (step) {  // 4-5 fused: conv step + SiLU + requant with the frozen exponents
            ep.conv_w_q = W->conv_w_q;
            ep.conv_p_w = W->conv_p_w;
            ep.conv_b_q16 = W->conv_b_q16;
            ep.conv_p = pdev;
            ep.conv_state = cache->conv_state;
            ep.x_out = w.x_q;
            ep.b_out = w.b_q;
            ep.c_out = w.c_q;
            ep.xbc_q = keep ? w.xbc_q : nullptr;
            ep.conv_amax_slots = w.slots + kRegionConvX * kSlotRegionWords;
            ep.d_inner = di;
            ep.dstate = N;
            ep.sz_out = w.sz;
            ep.write_xbc = keep;
            ep.dt_bias = W->dt_bias;  // 6 fused: dt and the decay for the scan step
            ep.a_q16 = W->a_q16;
            ep.dt_out = w.dt;
            ep.da_out = w.da;
        }
        if ((st = gemm_run(w.u_q, W->w_in_q, T, dip, dm, ep, s)) != FM_OK) return st;
    }
    if ((st = mark(2)) != FM_OK) return st;
    // 4-5. conv1d + SiLU + requant of x / B / C
    if (!step) {
        ConvArgs a{};
        a.xbc = w.v + di;
        a.xbc_stride = dip;
        a.batch = batch;
        a.len = len;
        a.d_inner = di;
        a.dstate = N;
        a.w_q = W->conv_w_q;
        a.p_w = W->conv_p_w;
        a.b_q16 = W->conv_b_q16;
        a.xbc_amax = small_f + kAmaxXbc;
        a.xbc_amax_slots = w.slots + kRegionXbc * kSlotRegionWords;
        const bool fixed_p = stat || decode;
        a.p_fixed = fixed_p ? pdev : nullptr;
        a.state_in = decode ? cache->conv_state : nullptr;
        a.state_out = cache ? cache->conv_state : nullptr;
        a.xbc_q = keep ? w.xbc_q : nullptr;
        a.s16 = w.s16;
        a.amax_q16 = small_i + kAmaxQ;
        a.amax_slots = w.slots + kRegionConvX * kSlotRegionWords;
        a.x_out = w.x_q;
        a.b_out = w.b_q;
        a.c_out = w.c_q;
        a.p_out = pdev;
        // with fixed exponents the conv kernel records the maxima itself (calibration stats)
        a.amax_stats = fixed_p ? small_i + kAmaxXbc : nullptr;
        // the scan's dt / decay prologue rides along (a6)
        a.dt_raw = w.v + di + ch;
        a.dt_stride = dip;
        a.dt_bias = W->dt_bias;
        a.a_q16 = W->a_q16;
        a.nheads = H;
        a.dt_out = w.dt;
        a.da_out = w.da;
        a.qs = qs;
        if ((st = conv_run(a, s)) != FM_OK) return st;
    }
    // 6-7. dt / decay and the scan
    {
        ScanArgs a{};
        a.x = w.x_q;
        a.bm = w.b_q;
        a.cm = w.c_q;
        a.dt_raw = w.v + di + ch;
        a.dt_stride = dip;
        a.dt_bias = W->dt_bias;
        a.a_q16 = W->a_q16;
        a.d_q16 = W->d_q16;
        a.p = pdev;
        a.batch = batch;
        a.len = len;
        a.nheads = H;
        a.headdim = P;
        a.dstate = N;
        a.state_in = decode ? cache->ssm_state : nullptr;
        a.state_out = cache ? cache->ssm_state : nullptr;
        a.y = w.y;
        a.dt_out = w.dt;
        a.da_out = w.da;
        a.dt_ready = true;  // formed by the conv launch, or by in_proj's epilogue (step)
        a.state_bits = decode ? state_bits : 32;
        a.state_shift = decode ? state_shift : 0;
        hipEvent_t ev0 = opts.ev[3], ev1 = opts.ev[4];
        if (ssd_ws && !decode) {
            if ((st = ssd_run(a, ssd_ws, s, ev0, ev1)) != FM_OK) return st;
        } else if ((st = scan_run(a, w.scan_ws, s, ev0, ev1)) != FM_OK) {
            return st;
        }
    }
    // 8. gate + RMSNorm + rotate + quantize the out_proj input
    {
        GateArgs g{};
        g.y = w.y;
        g.z = w.v;
        g.z_stride = dip;
        g.p = pdev;
        g.norm_w = W->norm_w;
        g.rows = T;
        g.d_inner = di;
        g.mode = mode;
        g.scoe = stat ? sp->scoe[1] : 0;
        g.sshift = stat ? sp->sshift[1] : 0;
        g.q = w.g_q;
        g.scale_out = small_f + kScaleG;
        g.amax_stats = stat ? small_f + kAmaxG : nullptr;
        g.normed_out = keep ? w.normed : nullptr;
        g.rot_ws = w.rot;
        g.amax_ws = small_f + kAmaxG;
        g.amax_slots = w.slots + kRegionG * kSlotRegionWords;
        g.rowmax = step ? w.rowmax + 64 : nullptr;
        g.step_slots = step ? w.slots : nullptr;
        g.step_small = step ? w.small : nullptr;
        g.sz = step ? w.sz : nullptr;
        g.qs = qs;
        if ((st = gate_run(g, s)) != FM_OK) return st;
    }
    // 9. out_proj W8A8 (+ residual for stacks)
    {
        GemmEpilogue ep;
        ep.out = out;
        ep.ld_out = dm;
        ep.s_a = small_f + kScaleG;
        ep.s_b = W->s_w_out;
        if (d->prenorm_residual) {
            ep.resid = u;
            ep.ld_resid = dm;
        }
        // one-token step: the codes of the rotated gate rows with the tensor scale,
        // formed once (the product then reads int8 A)
        if (step && (st = quant_rows_run(w.rot, w.rowmax + 64, T, di, mode,
                                         stat ? sp->scoe[1] : 0, stat ? sp->sshift[1] : 0, w.g_q,
                                         small_f + kScaleG, small_f + kAmaxG, s)) != FM_OK)
            return st;
        if ((st = mark(5)) != FM_OK) return st;
        // the call's scales, exponents and statistics go out with this last kernel
        ep.pub_small = w.small;
        ep.pub_qp = qp;
        ep.pub_cache_p = (cache && !decode) ? cache->p : nullptr;
        if ((st = gemm_run(w.g_q, W->w_out_q, T, dm, di, ep, s)) != FM_OK) return st;
        return mark(6);
    }
}

// ---------------------------------------------------------------- preparation
__global__ void prep_conv_kernel(const float* __restrict__ w, const float* __restrict__ b,
                                 int64_t ch, int8_t* w_q, int32_t* p_w, int32_t* b_q16) {
    const int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= ch) return;
    float m = 0.0f;
    for (int k = 0; k < 4; ++k) m = fmaxf(m, fabsf(w[c * 4 + k]));
    const int p = pot_from_f32(m);
    const float sc = ldexpf(1.0f, p);
    for (int k = 0; k < 4; ++k)
        w_q[c * 4 + k] = (int8_t)fminf(fmaxf(rintf(w[c * 4 + k] * sc), -127.0f), 127.0f);
    p_w[c] = p;
    b_q16[c] = f2i_sat(rintf(b[c] * 65536.0f));
}

__global__ void prep_q16_kernel(const float* __restrict__ a, const float* __restrict__ dv,
                                int64_t h, int32_t* a_q16, int32_t* d_q16) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= h) return;
    a_q16[i] = f2i_sat(rintf(a[i] * 65536.0f));
    d_q16[i] = f2i_sat(rintf(dv[i] * 65536.0f));
}

fm_status prepare_run(const fm_layer_desc* d, const float* w_in, const float* w_out,
                      const float* conv_w, const float* conv_b, const float* a, const float* dv,
                      int8_t* w_in_q, float* s_w_in, int8_t* w_out_q, float* s_w_out,
                      int8_t* conv_w_q, int32_t* conv_p_w, int32_t* conv_b_q16, int32_t* a_q16,
                      int32_t* d_q16, void* ws, hipStream_t s) {
    const int64_t dm = d->d_model, di = d->d_inner, N = d->dstate, H = d->nheads;
    const int64_t ch = di + 2 * N, dip = 2 * di + 2 * N + H;
    // two maxima, then one slot region for each
    float* amax = (float*)ws;
    int32_t* slots = (int32_t*)((char*)ws + 256);
    fm_status st;
    if ((st = zero_words(ws, 64 + 2 * kSlotRegionWords, s)) != FM_OK) return st;
    if ((st = hq_run(w_in, dip, dm, FM_SCALE_DYNAMIC, 0, 0, w_in_q, s_w_in, nullptr, amax, slots,
                     s)) != FM_OK)
        return st;
    if ((st = hq_run(w_out, dm, di, FM_SCALE_DYNAMIC, 0, 0, w_out_q, s_w_out, nullptr, amax + 1,
                     slots + kSlotRegionWords, s)) != FM_OK)
        return st;
    prep_conv_kernel<<<(unsigned)((ch + 255) / 256), 256, 0, s>>>(conv_w, conv_b, ch, conv_w_q,
                                                                 conv_p_w, conv_b_q16);
    if ((st = check_launch("prep_conv_kernel")) != FM_OK) return st;
    prep_q16_kernel<<<(unsigned)((H + 255) / 256), 256, 0, s>>>(a, dv, H, a_q16, d_q16);
    return check_launch("prep_q16_kernel");
}

}  // namespace fm
