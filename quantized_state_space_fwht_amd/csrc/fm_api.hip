// Public C-ABI entry points (include/fm.h): argument validation on the host,
// then the launches.  On any validation error nothing is launched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "fm_internal.hpp"

namespace fm {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
}

fm_status fail(fm_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return s;
}

int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

fm_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(FM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return FM_OK;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

static fm_status check_ws(void* ws, size_t have, size_t need, const char* who) {
    if (need == 0) return FM_OK;
    if (!ws) return fail(FM_ERR_WORKSPACE, "%s: workspace is NULL (%zu bytes needed)", who, need);
    if (have < need)
        return fail(FM_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who, have, need);
    if (!aligned(ws, 256)) return fail(FM_ERR_WORKSPACE, "%s: workspace not 256-byte aligned", who);
    return FM_OK;
}

static fm_status check_layer_desc(const fm_layer_desc* d, const char* who) {
    if (!d) return fail(FM_ERR_NULL, "%s: desc is NULL", who);
    if (d->d_conv != 4) return fail(FM_ERR_SHAPE, "%s: d_conv must be 4", who);
    if (d->d_model <= 0 || d->d_model % 256 || d->d_model > 16384)
        return fail(FM_ERR_SHAPE, "%s: d_model must be a multiple of 256 in (0, 16384]", who);
    if (d->d_inner <= 0 || d->d_inner % 256 || d->d_inner > 8192)
        return fail(FM_ERR_SHAPE, "%s: d_inner must be a multiple of 256 in (0, 8192]", who);
    if (d->headdim <= 0 || d->headdim % 8 || d->nheads * d->headdim != d->d_inner)
        return fail(FM_ERR_SHAPE, "%s: nheads * headdim must equal d_inner, headdim %% 8 == 0", who);
    if (d->dstate != 64 && d->dstate != 128)
        return fail(FM_ERR_SHAPE, "%s: dstate must be 64 or 128", who);
    if (d->mode != FM_SCALE_DYNAMIC && d->mode != FM_SCALE_STATIC)
        return fail(FM_ERR_MODE, "%s: bad mode %d", who, d->mode);
    return FM_OK;
}

static fm_status check_static_hq(int32_t scoe, int32_t sshift, const char* who) {
    if (scoe <= 0 || scoe >= (1 << 24))
        return fail(FM_ERR_MODE, "%s: scoe %d outside (0, 2^24)", who, scoe);
    if (sshift < -126 || sshift > 126)
        return fail(FM_ERR_MODE, "%s: sshift %d outside [-126, 126]", who, sshift);
    return FM_OK;
}

static fm_status check_static_params(const fm_static_params* sp, const char* who) {
    if (!sp) return fail(FM_ERR_NULL, "%s: static mode needs static params", who);
    fm_status st;
    for (int i = 0; i < 2; ++i)
        if ((st = check_static_hq(sp->scoe[i], sp->sshift[i], who)) != FM_OK) return st;
    for (int i = 0; i < 4; ++i)
        if (sp->p[i] < FM_PMIN || sp->p[i] > FM_PMAX)
            return fail(FM_ERR_MODE, "%s: exponent p[%d] = %d outside [%d, %d]", who, i, sp->p[i],
                        FM_PMIN, FM_PMAX);
    return FM_OK;
}

static fm_status check_weights(const fm_layer_weights* w, const char* who) {
    if (!w) return fail(FM_ERR_NULL, "%s: weights is NULL", who);
    if (!w->w_in_q || !w->s_w_in || !w->w_out_q || !w->s_w_out || !w->conv_w_q || !w->conv_p_w ||
        !w->conv_b_q16 || !w->dt_bias || !w->a_q16 || !w->d_q16 || !w->norm_w)
        return fail(FM_ERR_NULL, "%s: a weight pointer is NULL", who);
    if (!aligned(w->w_in_q, 16) || !aligned(w->w_out_q, 16) || !aligned(w->norm_w, 16))
        return fail(FM_ERR_SHAPE, "%s: weight arrays must be 16-byte aligned", who);
    return FM_OK;
}

}  // namespace fm

using namespace fm;

extern "C" {

int fm_abi_version(void) { return FM_ABI_VERSION; }

const char* fm_status_string(fm_status s) {
    switch (s) {
        case FM_OK: return "ok";
        case FM_ERR_NULL: return "null pointer";
        case FM_ERR_SHAPE: return "unsupported shape";
        case FM_ERR_MODE: return "bad mode or static parameters";
        case FM_ERR_WORKSPACE: return "workspace missing or too small";
        case FM_ERR_HIP: return "HIP launch failed";
    }
    return "unknown status";
}

const char* fm_last_error(void) { return g_err; }

// ---------------------------------------------------------------- fm_hadamard_quant
size_t fm_hadamard_quant_workspace_size(int64_t rows, int64_t k) {
    (void)rows;
    (void)k;
    return 256 + kSlotRegionWords * sizeof(int32_t);  // the maximum, then its slot region
}

fm_status fm_hadamard_quant(const float* x, int64_t rows, int64_t k, fm_scale_mode mode,
                            int32_t scoe, int32_t sshift, int8_t* q, float* scale_out,
                            float* amax_stats, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
    const char* who = "fm_hadamard_quant";
    g_err[0] = 0;
    if (!scale_out) return fail(FM_ERR_NULL, "%s: scale_out is NULL", who);
    if (rows < 0 || k <= 0 || k % 256 || k > 65536 || rows * k >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE, "%s: need k a positive multiple of 256 (<= 65536), rows >= 0, "
                    "rows*k < 2^31 (rows=%lld k=%lld)", who, (long long)rows, (long long)k);
    if (rows > 0 && (!x || !q)) return fail(FM_ERR_NULL, "%s: x or q is NULL", who);
    if (rows > 0 && (!aligned(x, 16) || !aligned(q, 4)))
        return fail(FM_ERR_SHAPE, "%s: x must be 16-byte and q 4-byte aligned", who);
    fm_status st;
    if (mode == FM_SCALE_DYNAMIC) {
        const size_t need = fm_hadamard_quant_workspace_size(rows, k);
        if ((st = check_ws(workspace, workspace_bytes, need, who)) != FM_OK) return st;
        if ((st = zero_words(workspace, 64 + kSlotRegionWords, stream)) != FM_OK) return st;
        return hq_run(x, rows, k, mode, 0, 0, q, scale_out, amax_stats, (float*)workspace,
                      (int32_t*)((char*)workspace + 256), stream);
    }
    if (mode != FM_SCALE_STATIC) return fail(FM_ERR_MODE, "%s: bad mode %d", who, (int)mode);
    if ((st = check_static_hq(scoe, sshift, who)) != FM_OK) return st;
    return hq_run(x, rows, k, mode, scoe, sshift, q, scale_out, amax_stats, nullptr, nullptr,
                  stream);
}

// ---------------------------------------------------------------- fm_w8a8_gemm
fm_status fm_w8a8_gemm(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k,
                       const float* scale_a, const float* scale_b, int32_t* acc, float* out,
                       hipStream_t stream) {
    const char* who = "fm_w8a8_gemm";
    g_err[0] = 0;
    if (!acc && !out) return fail(FM_ERR_NULL, "%s: both acc and out are NULL", who);
    if (out && (!scale_a || !scale_b)) return fail(FM_ERR_NULL, "%s: out needs both scales", who);
    if (m < 0 || n < 0 || k <= 0 || k % 64 || k > 131072 || m > ((int64_t)1 << 24) ||
        n > ((int64_t)1 << 24))
        return fail(FM_ERR_SHAPE, "%s: need k a positive multiple of 64 (<= 131072), "
                    "0 <= m, n <= 2^24 (m=%lld n=%lld k=%lld)", who, (long long)m, (long long)n,
                    (long long)k);
    if (m > 0 && n > 0) {
        if (!a || !b) return fail(FM_ERR_NULL, "%s: a or b is NULL", who);
        if (!aligned(a, 16) || !aligned(b, 16))
            return fail(FM_ERR_SHAPE, "%s: a and b must be 16-byte aligned", who);
    }
    GemmEpilogue ep;
    ep.acc = acc;
    ep.ld_acc = n;
    ep.out = out;
    ep.ld_out = n;
    ep.s_a = scale_a;
    ep.s_b = scale_b;
    return gemm_run(a, b, m, n, k, ep, stream);
}

// ---------------------------------------------------------------- fm_conv1d_pot
size_t fm_conv1d_pot_workspace_size(int64_t batch, int64_t len, int64_t d_inner, int64_t dstate) {
    if (batch < 0 || len < 0 || d_inner < 0 || dstate < 0) return 0;
    return 256 + 4 * kSlotRegionWords * sizeof(int32_t) +
           align256((size_t)(batch * len * (d_inner + 2 * dstate)) * sizeof(int32_t));
}

fm_status fm_conv1d_pot(const float* xbc, int64_t xbc_row_stride, int64_t batch, int64_t len,
                        int64_t d_inner, int64_t dstate, const int8_t* w_q, const int32_t* p_w,
                        const int32_t* b_q16, fm_scale_mode mode, const int32_t* p_fixed,
                        const int8_t* conv_state_in, int8_t* conv_state_out, int8_t* xbc_q,
                        int8_t* x_out, int8_t* b_out, int8_t* c_out, int32_t* p_out,
                        int32_t* amax_stats, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
    const char* who = "fm_conv1d_pot";
    g_err[0] = 0;
    if (batch < 1 || len < 1 || d_inner <= 0 || d_inner % 64 || dstate <= 0 || dstate % 64)
        return fail(FM_ERR_SHAPE, "%s: need batch, len >= 1 and d_inner, dstate positive "
                    "multiples of 64", who);
    const int64_t ch = d_inner + 2 * dstate;
    if (xbc_row_stride < ch) return fail(FM_ERR_SHAPE, "%s: row stride < channels", who);
    if (batch * len * ch >= ((int64_t)1 << 31) || batch > 65535 || ch / 64 > 65535)
        return fail(FM_ERR_SHAPE, "%s: tensor too large", who);
    if (!xbc || !w_q || !p_w || !b_q16 || !x_out || !b_out || !c_out || !p_out)
        return fail(FM_ERR_NULL, "%s: a required pointer is NULL", who);
    if (!aligned(x_out, 4) || !aligned(b_out, 4) || !aligned(c_out, 4))
        return fail(FM_ERR_SHAPE, "%s: outputs must be 4-byte aligned", who);
    if (conv_state_in && conv_state_in == conv_state_out && len > 16)
        return fail(FM_ERR_SHAPE, "%s: conv_state_in may alias conv_state_out only for len <= 16",
                    who);
    ConvArgs a{};
    a.xbc = xbc;
    a.xbc_stride = xbc_row_stride;
    a.batch = batch;
    a.len = len;
    a.d_inner = d_inner;
    a.dstate = dstate;
    a.w_q = w_q;
    a.p_w = p_w;
    a.b_q16 = b_q16;
    a.state_in = conv_state_in;
    a.state_out = conv_state_out;
    a.xbc_q = xbc_q;
    a.x_out = x_out;
    a.b_out = b_out;
    a.c_out = c_out;
    a.p_out = p_out;
    a.amax_stats = amax_stats;
    fm_status st;
    if (mode == FM_SCALE_STATIC) {
        if (!p_fixed) return fail(FM_ERR_NULL, "%s: static mode needs p_fixed", who);
        a.p_fixed = p_fixed;
        return conv_run(a, stream);
    }
    if (mode != FM_SCALE_DYNAMIC) return fail(FM_ERR_MODE, "%s: bad mode %d", who, (int)mode);
    const size_t need = fm_conv1d_pot_workspace_size(batch, len, d_inner, dstate);
    if ((st = check_ws(workspace, workspace_bytes, need, who)) != FM_OK) return st;
    float* amax_x = (float*)workspace;           // word 0: max|xBC|
    int32_t* amax_q = (int32_t*)workspace + 1;   // words 1..3: the part maxima
    a.xbc_amax = amax_x;
    a.amax_q16 = amax_q;
    // slot regions: x, B, C maxima, then max |xBC|
    a.amax_slots = (int32_t*)((char*)workspace + 256);
    int32_t* xbc_slots = a.amax_slots + 3 * kSlotRegionWords;
    a.xbc_amax_slots = xbc_slots;
    a.s16 = (int32_t*)((char*)workspace + 256 + 4 * kSlotRegionWords * sizeof(int32_t));
    if ((st = zero_words(workspace, 64 + 4 * kSlotRegionWords, stream)) != FM_OK) return st;
    if ((st = amax_strided_run(xbc, batch * len, ch, xbc_row_stride, xbc_slots, stream)) != FM_OK)
        return st;
    return conv_run(a, stream);
}

// ---------------------------------------------------------------- fm_ssm_scan_pot
size_t fm_ssm_scan_pot_workspace_size(int64_t batch, int64_t len, int64_t dstate) {
    if (batch < 0 || len < 0 || dstate < 0) return 0;
    return scan_ws_bytes(batch, len, dstate);
}

static fm_status scan_args(const char* who, const int8_t* x, const int8_t* bm, const int8_t* cm,
                           const float* dt_raw, int64_t dt_row_stride, const float* dt_bias,
                           const int32_t* a_q16, const int32_t* d_q16, const int32_t* p,
                           int64_t batch, int64_t len, int64_t nheads, int64_t headdim,
                           int64_t dstate, const int32_t* state_in, int32_t* state_out, int32_t* y,
                           int32_t* dt_out, int32_t* da_out, ScanArgs* out) {
    if (!x || !bm || !cm || !dt_raw || !dt_bias || !a_q16 || !d_q16 || !p || !y || !dt_out ||
        !da_out)
        return fail(FM_ERR_NULL, "%s: a required pointer is NULL", who);
    if (batch < 1 || len < 1 || nheads < 1 || headdim < 8 || headdim % 8 ||
        (dstate != 64 && dstate != 128) || batch > 65535 || nheads > 65535 ||
        batch * len * nheads * headdim >= ((int64_t)1 << 31) ||
        batch * len * dstate >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE,
                    "%s: need headdim %% 8 == 0, dstate in {64, 128}, batch*len*nheads*headdim "
                    "and batch*len*dstate below 2^31", who);
    if (dt_row_stride < nheads) return fail(FM_ERR_SHAPE, "%s: dt row stride < nheads", who);
    if (!aligned(y, 8) || !aligned(x, 2) || !aligned(bm, 16) || !aligned(cm, 16))
        return fail(FM_ERR_SHAPE, "%s: y must be 8-byte, x 2-byte, bm / cm 16-byte aligned", who);
    ScanArgs a{};
    a.x = x;
    a.bm = bm;
    a.cm = cm;
    a.dt_raw = dt_raw;
    a.dt_stride = dt_row_stride;
    a.dt_bias = dt_bias;
    a.a_q16 = a_q16;
    a.d_q16 = d_q16;
    a.p = p;
    a.batch = batch;
    a.len = len;
    a.nheads = nheads;
    a.headdim = headdim;
    a.dstate = dstate;
    a.state_in = state_in;
    a.state_out = state_out;
    a.y = y;
    a.dt_out = dt_out;
    a.da_out = da_out;
    *out = a;
    return FM_OK;
}

fm_status fm_ssm_scan_pot(const int8_t* x, const int8_t* bm, const int8_t* cm,
                          const float* dt_raw, int64_t dt_row_stride, const float* dt_bias,
                          const int32_t* a_q16, const int32_t* d_q16, const int32_t* p,
                          int64_t batch, int64_t len, int64_t nheads, int64_t headdim,
                          int64_t dstate, const int32_t* state_in, int32_t* state_out, int32_t* y,
                          int32_t* dt_out, int32_t* da_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_ssm_scan_pot";
    g_err[0] = 0;
    ScanArgs a;
    fm_status st = scan_args(who, x, bm, cm, dt_raw, dt_row_stride, dt_bias, a_q16, d_q16, p,
                             batch, len, nheads, headdim, dstate, state_in, state_out, y, dt_out,
                             da_out, &a);
    if (st != FM_OK) return st;
    if ((st = check_ws(workspace, workspace_bytes, scan_ws_bytes(batch, len, dstate), who)) !=
        FM_OK)
        return st;
    return scan_run(a, workspace, stream);
}

size_t fm_ssm_scan_ssd_workspace_size(int64_t batch, int64_t len, int64_t nheads,
                                      int64_t headdim, int64_t dstate) {
    if (batch < 1 || len < 1 || nheads < 1 || headdim < 1 || dstate < 1) return 0;
    return ssd_ws_bytes(batch, len, nheads, headdim, dstate);
}

fm_status fm_ssm_scan_ssd(const int8_t* x, const int8_t* bm, const int8_t* cm,
                          const float* dt_raw, int64_t dt_row_stride, const float* dt_bias,
                          const int32_t* a_q16, const int32_t* d_q16, const int32_t* p,
                          int64_t batch, int64_t len, int64_t nheads, int64_t headdim,
                          int64_t dstate, const int32_t* state_in, int32_t* state_out, int32_t* y,
                          int32_t* dt_out, int32_t* da_out, void* workspace,
                          size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_ssm_scan_ssd";
    g_err[0] = 0;
    ScanArgs a;
    fm_status st = scan_args(who, x, bm, cm, dt_raw, dt_row_stride, dt_bias, a_q16, d_q16, p,
                             batch, len, nheads, headdim, dstate, state_in, state_out, y, dt_out,
                             da_out, &a);
    if (st != FM_OK) return st;
    if (headdim != 64) return fail(FM_ERR_SHAPE, "%s: headdim must be 64", who);
    if (!aligned(x, 16)) return fail(FM_ERR_SHAPE, "%s: x must be 16-byte aligned", who);
    if ((st = check_ws(workspace, workspace_bytes,
                       ssd_ws_bytes(batch, len, nheads, headdim, dstate), who)) != FM_OK)
        return st;
    return ssd_run(a, workspace, stream);
}

// ---------------------------------------------------------------- fm_nau_eval
fm_status fm_nau_eval(fm_nau_fn fn, const int32_t* x, int32_t* y, int64_t n, hipStream_t stream) {
    const char* who = "fm_nau_eval";
    g_err[0] = 0;
    if (fn != FM_NAU_EXP && fn != FM_NAU_SOFTPLUS && fn != FM_NAU_SILU)
        return fail(FM_ERR_MODE, "%s: bad function %d", who, (int)fn);
    if (n < 0) return fail(FM_ERR_SHAPE, "%s: n < 0", who);
    if (n > 0 && (!x || !y)) return fail(FM_ERR_NULL, "%s: x or y is NULL", who);
    return nau_run((int)fn, x, y, n, stream);
}

fm_status fm_nau_eval_knots(fm_nau_fn fn, const int64_t* knots_q30, const int32_t* x, int32_t* y,
                            int64_t n, hipStream_t stream) {
    const char* who = "fm_nau_eval_knots";
    g_err[0] = 0;
    if (fn != FM_NAU_EXP && fn != FM_NAU_SOFTPLUS && fn != FM_NAU_SILU)
        return fail(FM_ERR_MODE, "%s: bad function %d", who, (int)fn);
    if (!knots_q30) return fail(FM_ERR_NULL, "%s: knots is NULL", who);
    // bounds of the exact float64 evaluation: products below 2^53 for knots
    // under 2^32, and the exponent clamp at -18 needs Y[0] < 2^31
    for (int i = 0; i < 9; ++i)
        if (knots_q30[i] <= ((int64_t)1 << 29) || knots_q30[i] >= ((int64_t)1 << 32) ||
            (i == 0 && knots_q30[0] >= ((int64_t)1 << 31)))
            return fail(FM_ERR_SHAPE, "%s: knot %d = %lld outside (2^29, 2^32) (knot 0: < 2^31)",
                        who, i, (long long)knots_q30[i]);
    if (n < 0) return fail(FM_ERR_SHAPE, "%s: n < 0", who);
    if (n > 0 && (!x || !y)) return fail(FM_ERR_NULL, "%s: x or y is NULL", who);
    return nau_run((int)fn, x, y, n, stream, knots_q30);
}

// ---------------------------------------------------------------- fm_gate_norm_quant
size_t fm_gate_norm_quant_workspace_size(int64_t rows, int64_t d_inner) {
    if (rows < 0 || d_inner < 0) return 0;
    return 256 + kSlotRegionWords * sizeof(int32_t) +
           align256((size_t)(rows * d_inner) * sizeof(float));
}

fm_status fm_gate_norm_quant(const int32_t* y, const float* z, int64_t z_row_stride,
                             const int32_t* p, const float* norm_w, int64_t rows, int64_t d_inner,
                             fm_scale_mode mode, int32_t scoe, int32_t sshift, int8_t* q,
                             float* scale_out, float* amax_stats, float* normed_out,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_gate_norm_quant";
    g_err[0] = 0;
    if (!scale_out) return fail(FM_ERR_NULL, "%s: scale_out is NULL", who);
    if (rows < 0 || d_inner <= 0 || d_inner % 256 || d_inner > 8192 ||
        rows * d_inner >= ((int64_t)1 << 31) || rows > ((int64_t)1 << 30))
        return fail(FM_ERR_SHAPE, "%s: need d_inner a multiple of 256 in (0, 8192]", who);
    if (rows > 0 && (!y || !z || !p || !norm_w || !q))
        return fail(FM_ERR_NULL, "%s: a required pointer is NULL", who);
    if (z_row_stride < d_inner) return fail(FM_ERR_SHAPE, "%s: z row stride < d_inner", who);
    if (!aligned(norm_w, 16) || !aligned(q, 4) || (normed_out && !aligned(normed_out, 16)))
        return fail(FM_ERR_SHAPE, "%s: norm_w / normed_out 16-byte, q 4-byte aligned", who);
    GateArgs g{};
    g.y = y;
    g.z = z;
    g.z_stride = z_row_stride;
    g.p = p;
    g.norm_w = norm_w;
    g.rows = rows;
    g.d_inner = d_inner;
    g.mode = mode;
    g.q = q;
    g.scale_out = scale_out;
    g.amax_stats = amax_stats;
    g.normed_out = normed_out;
    fm_status st;
    if (mode == FM_SCALE_STATIC) {
        if ((st = check_static_hq(scoe, sshift, who)) != FM_OK) return st;
        g.scoe = scoe;
        g.sshift = sshift;
        return gate_run(g, stream);
    }
    if (mode != FM_SCALE_DYNAMIC) return fail(FM_ERR_MODE, "%s: bad mode %d", who, (int)mode);
    const size_t need = fm_gate_norm_quant_workspace_size(rows, d_inner);
    if ((st = check_ws(workspace, workspace_bytes, need, who)) != FM_OK) return st;
    g.amax_ws = (float*)workspace;
    g.amax_slots = (int32_t*)((char*)workspace + 256);  // one slot region
    g.rot_ws = (float*)((char*)workspace + 256 + kSlotRegionWords * sizeof(int32_t));
    if ((st = zero_words(workspace, 64 + kSlotRegionWords, stream)) != FM_OK) return st;
    return gate_run(g, stream);
}

// ---------------------------------------------------------------- layer
size_t fm_prepare_layer_workspace_size(const fm_layer_desc* d) {
    (void)d;
    return 256 + 2 * kSlotRegionWords * sizeof(int32_t);  // two maxima, two slot regions
}

fm_status fm_prepare_layer(const fm_layer_desc* d, const float* w_in, const float* w_out,
                           const float* conv_w, const float* conv_b, const float* a,
                           const float* dvec, int8_t* w_in_q, float* s_w_in, int8_t* w_out_q,
                           float* s_w_out, int8_t* conv_w_q, int32_t* conv_p_w,
                           int32_t* conv_b_q16, int32_t* a_q16, int32_t* d_q16, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_prepare_layer";
    g_err[0] = 0;
    fm_status st;
    if ((st = check_layer_desc(d, who)) != FM_OK) return st;
    if (!w_in || !w_out || !conv_w || !conv_b || !a || !dvec || !w_in_q || !s_w_in || !w_out_q ||
        !s_w_out || !conv_w_q || !conv_p_w || !conv_b_q16 || !a_q16 || !d_q16)
        return fail(FM_ERR_NULL, "%s: a required pointer is NULL", who);
    if (!aligned(w_in, 16) || !aligned(w_out, 16) || !aligned(w_in_q, 4) || !aligned(w_out_q, 4))
        return fail(FM_ERR_SHAPE, "%s: weights 16-byte, codes 4-byte aligned", who);
    if ((st = check_ws(workspace, workspace_bytes, fm_prepare_layer_workspace_size(d), who)) !=
        FM_OK)
        return st;
    return prepare_run(d, w_in, w_out, conv_w, conv_b, a, dvec, w_in_q, s_w_in, w_out_q, s_w_out,
                       conv_w_q, conv_p_w, conv_b_q16, a_q16, d_q16, workspace, stream);
}

size_t fm_mamba2_layer_workspace_size(const fm_layer_desc* d, int64_t batch, int64_t len) {
    if (!d || batch < 0 || len < 0) return 0;
    return layer_ws_bytes(d, batch, len);
}

// every argument of a layer call but the workspace
static fm_status check_layer_args(const fm_layer_desc* d, const fm_layer_weights* w,
                                  const fm_static_params* sp, const float* u, int64_t batch,
                                  int64_t len, const float* out, fm_qparams* qp, const char* who,
                                  bool ssd) {
    fm_status st;
    if ((st = check_layer_desc(d, who)) != FM_OK) return st;
    if ((st = check_weights(w, who)) != FM_OK) return st;
    if (d->mode == FM_SCALE_STATIC && (st = check_static_params(sp, who)) != FM_OK) return st;
    if (!u || !out || !qp) return fail(FM_ERR_NULL, "%s: u, out or qp is NULL", who);
    if (u == out) return fail(FM_ERR_SHAPE, "%s: out may not alias u", who);
    if (!aligned(u, 16) || !aligned(out, 16))
        return fail(FM_ERR_SHAPE, "%s: u and out must be 16-byte aligned", who);
    const int64_t T = batch * len;
    const int64_t dip = 2 * d->d_inner + 2 * d->dstate + d->nheads;
    if (batch < 1 || len < 1 || batch > 65535 || T > ((int64_t)1 << 24) ||
        T * dip >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE, "%s: batch=%lld len=%lld out of range", who, (long long)batch,
                    (long long)len);
    if (ssd && d->headdim != 64) return fail(FM_ERR_SHAPE, "%s: headdim must be 64", who);
    return FM_OK;
}

static fm_status check_layer_call(const fm_layer_desc* d, const fm_layer_weights* w,
                                  const fm_static_params* sp, const float* u, int64_t batch,
                                  int64_t len, const float* out, fm_qparams* qp, void* ws,
                                  size_t ws_bytes, const char* who, bool ssd = false) {
    fm_status st = check_layer_args(d, w, sp, u, batch, len, out, qp, who, ssd);
    if (st != FM_OK) return st;
    return check_ws(ws, ws_bytes,
                    ssd ? fm_mamba2_layer_workspace_size_ssd(d, batch, len)
                        : fm_mamba2_layer_workspace_size(d, batch, len),
                    who);
}

// Per-call options: everything off when NULL; validated before any launch.
static fm_status check_opts(const fm_layer_opts* o, bool decode, LayerOpts* out, const char* who) {
    *out = LayerOpts{};
    if (!o) return FM_OK;
    if (o->keep_intermediates != 0 && o->keep_intermediates != 1)
        return fail(FM_ERR_MODE, "%s: opts.keep_intermediates %d not 0 or 1", who,
                    o->keep_intermediates);
    if (o->reserved != 0) return fail(FM_ERR_MODE, "%s: opts.reserved must be 0", who);
    if (o->quant_stats) {
        if (decode) return fail(FM_ERR_MODE, "%s: decode calls do not collect quant_stats", who);
        if (!aligned(o->quant_stats, 8))
            return fail(FM_ERR_SHAPE, "%s: opts.quant_stats must be 8-byte aligned", who);
    }
    out->keep = o->keep_intermediates != 0;
    out->qs = o->quant_stats;
    if (o->stage_events)
        for (int i = 0; i < FM_LAYER_EVENTS; ++i) out->ev[i] = (hipEvent_t)o->stage_events[i];
    return FM_OK;
}

fm_status fm_mamba2_layer_prefill(const fm_layer_desc* d, const fm_layer_weights* w,
                                  const fm_static_params* sp, const float* u, int64_t batch,
                                  int64_t len, float* out, const fm_cache* cache, fm_qparams* qp,
                                  const fm_layer_opts* opts, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_mamba2_layer_prefill";
    g_err[0] = 0;
    fm_status st = check_layer_call(d, w, sp, u, batch, len, out, qp, workspace, workspace_bytes,
                                    who);
    if (st != FM_OK) return st;
    if (cache && (!cache->conv_state || !cache->ssm_state || !cache->p))
        return fail(FM_ERR_NULL, "%s: cache has a NULL member", who);
    LayerOpts lo;
    if ((st = check_opts(opts, false, &lo, who)) != FM_OK) return st;
    return layer_run(d, w, sp, u, batch, len, out, cache, qp, workspace, false, stream, lo);
}

size_t fm_mamba2_layer_workspace_size_ssd(const fm_layer_desc* d, int64_t batch, int64_t len) {
    const size_t base = fm_mamba2_layer_workspace_size(d, batch, len);
    if (!base) return 0;
    return align256(base) + ssd_ws_bytes(batch, len, d->nheads, d->headdim, d->dstate);
}

fm_status fm_mamba2_layer_prefill_ssd(const fm_layer_desc* d, const fm_layer_weights* w,
                                      const fm_static_params* sp, const float* u, int64_t batch,
                                      int64_t len, float* out, const fm_cache* cache,
                                      fm_qparams* qp, const fm_layer_opts* opts, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_mamba2_layer_prefill_ssd";
    g_err[0] = 0;
    fm_status st = check_layer_call(d, w, sp, u, batch, len, out, qp, workspace, workspace_bytes,
                                    who, true);
    if (st != FM_OK) return st;
    if (cache && (!cache->conv_state || !cache->ssm_state || !cache->p))
        return fail(FM_ERR_NULL, "%s: cache has a NULL member", who);
    LayerOpts lo;
    if ((st = check_opts(opts, false, &lo, who)) != FM_OK) return st;
    void* ssd_ws = (char*)workspace + align256(fm_mamba2_layer_workspace_size(d, batch, len));
    return layer_run(d, w, sp, u, batch, len, out, cache, qp, workspace, false, stream, lo, 32, 0,
                     ssd_ws);
}

fm_status fm_mamba2_layer_decode(const fm_layer_desc* d, const fm_layer_weights* w,
                                 const fm_static_params* sp, const float* u_t, int64_t batch,
                                 const fm_cache* cache, float* out_t, fm_qparams* qp,
                                 const fm_layer_opts* opts, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_mamba2_layer_decode";
    g_err[0] = 0;
    fm_status st = check_layer_call(d, w, sp, u_t, batch, 1, out_t, qp, workspace,
                                    workspace_bytes, who);
    if (st != FM_OK) return st;
    if (!cache || !cache->conv_state || !cache->ssm_state || !cache->p)
        return fail(FM_ERR_NULL, "%s: decode needs a complete cache", who);
    LayerOpts lo;
    if ((st = check_opts(opts, true, &lo, who)) != FM_OK) return st;
    return layer_run(d, w, sp, u_t, batch, 1, out_t, cache, qp, workspace, true, stream, lo);
}

// ---------------------------------------------------------------- no-allocation decode
// The scratch of fm_mamba2_layer_decode_noalloc: one static array per GPU.  In host
// code its name is only a stand-in: the device address of each GPU's copy is taken
// once per device with hipGetSymbolAddress and used everywhere instead.
static __device__ __align__(256) unsigned char scratch[FM_DECODE_SCRATCH_BYTES];

static fm_status scratch_ptr(void** out, const char* who) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* ptr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(FM_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(FM_ERR_HIP, "%s: device %d beyond the %d the scratch table holds", who, dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(FM_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                        hipGetErrorString(e));
        ptr[dev] = p;
    }
    *out = ptr[dev];
    return FM_OK;
}

fm_status fm_mamba2_layer_decode_noalloc(const fm_layer_desc* d, const fm_layer_weights* w,
                                         const fm_static_params* sp, const float* u_t,
                                         int64_t batch, const fm_cache* cache, float* out_t,
                                         fm_qparams* qp, const fm_layer_opts* opts,
                                         hipStream_t stream) {
    const char* who = "fm_mamba2_layer_decode_noalloc";
    g_err[0] = 0;
    fm_status st = check_layer_args(d, w, sp, u_t, batch, 1, out_t, qp, who, false);
    if (st != FM_OK) return st;
    const size_t need = fm_mamba2_layer_workspace_size(d, batch, 1);
    if (need > FM_DECODE_SCRATCH_BYTES)
        return fail(FM_ERR_WORKSPACE, "%s: batch %lld needs %zu bytes of scratch, more than the "
                    "%u bytes this entry point holds", who, (long long)batch, need,
                    FM_DECODE_SCRATCH_BYTES);
    if (!cache || !cache->conv_state || !cache->ssm_state || !cache->p)
        return fail(FM_ERR_NULL, "%s: decode needs a complete cache", who);
    LayerOpts lo;
    if ((st = check_opts(opts, true, &lo, who)) != FM_OK) return st;
    void* ws = nullptr;
    if ((st = scratch_ptr(&ws, who)) != FM_OK) return st;
    return layer_run(d, w, sp, u_t, batch, 1, out_t, cache, qp, ws, true, stream, lo);
}

static fm_status check_state_fmt(int32_t bits, int32_t shift, const char* who) {
    if (bits != 16 && bits != 24) return fail(FM_ERR_SHAPE, "%s: state_bits %d not 16 or 24", who, bits);
    if (shift < 0 || shift > 32 - bits)
        return fail(FM_ERR_SHAPE, "%s: state_shift %d not in [0, %d]", who, shift, 32 - bits);
    return FM_OK;
}

fm_status fm_mamba2_layer_decode_narrow(const fm_layer_desc* d, const fm_layer_weights* w,
                                        const fm_static_params* sp, const float* u_t,
                                        int64_t batch, const fm_cache_narrow* cache, float* out_t,
                                        fm_qparams* qp, const fm_layer_opts* opts,
                                        void* workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
    const char* who = "fm_mamba2_layer_decode_narrow";
    g_err[0] = 0;
    fm_status st = check_layer_call(d, w, sp, u_t, batch, 1, out_t, qp, workspace,
                                    workspace_bytes, who);
    if (st != FM_OK) return st;
    if (!cache || !cache->conv_state || !cache->ssm_state || !cache->p)
        return fail(FM_ERR_NULL, "%s: decode needs a complete cache", who);
    if ((st = check_state_fmt(cache->state_bits, cache->state_shift, who)) != FM_OK) return st;
    if (!aligned(cache->ssm_state, 16))
        return fail(FM_ERR_SHAPE, "%s: ssm_state must be 16-byte aligned", who);
    LayerOpts lo;
    if ((st = check_opts(opts, true, &lo, who)) != FM_OK) return st;
    const fm_cache c32{cache->conv_state, (int32_t*)cache->ssm_state, cache->p};
    return layer_run(d, w, sp, u_t, batch, 1, out_t, &c32, qp, workspace, true, stream, lo,
                     cache->state_bits, cache->state_shift);
}

size_t fm_state_narrow_bytes(int64_t count, int32_t bits) {
    return count > 0 && (bits == 16 || bits == 24) ? (size_t)count * (size_t)(bits / 8) : 0;
}

fm_status fm_state_narrow(const int32_t* state, int64_t count, int32_t bits, int32_t shift,
                          void* codes, hipStream_t stream) {
    const char* who = "fm_state_narrow";
    g_err[0] = 0;
    fm_status st = check_state_fmt(bits, shift, who);
    if (st != FM_OK) return st;
    if (count < 0) return fail(FM_ERR_SHAPE, "%s: count %lld < 0", who, (long long)count);
    if (count > 0 && (!state || !codes)) return fail(FM_ERR_NULL, "%s: NULL pointer", who);
    return state_narrow_run(state, count, bits, shift, codes, stream);
}

fm_status fm_state_shift_for(uint32_t amax, int32_t bits, int32_t headroom, int32_t* shift) {
    const char* who = "fm_state_shift_for";
    g_err[0] = 0;
    if (!shift) return fail(FM_ERR_NULL, "%s: shift is NULL", who);
    if (bits != 16 && bits != 24) return fail(FM_ERR_SHAPE, "%s: bits %d not 16 or 24", who, bits);
    if (headroom < 0 || headroom > 32)
        return fail(FM_ERR_SHAPE, "%s: headroom %d not in [0, 32]", who, headroom);
    int need = headroom;  // bit length of amax, plus the headroom
    for (uint32_t a = amax; a; a >>= 1) ++need;
    int sh = need - (bits - 1);
    if (sh < 0) sh = 0;
    if (sh > 32 - bits) sh = 32 - bits;
    *shift = sh;
    return FM_OK;
}

fm_status fm_state_widen(const void* codes, int64_t count, int32_t bits, int32_t shift,
                         int32_t* state, hipStream_t stream) {
    const char* who = "fm_state_widen";
    g_err[0] = 0;
    fm_status st = check_state_fmt(bits, shift, who);
    if (st != FM_OK) return st;
    if (count < 0) return fail(FM_ERR_SHAPE, "%s: count %lld < 0", who, (long long)count);
    if (count > 0 && (!state || !codes)) return fail(FM_ERR_NULL, "%s: NULL pointer", who);
    return state_widen_run(codes, count, bits, shift, state, stream);
}

fm_status fm_state_absmax(const int32_t* state, int64_t count, uint32_t* amax, hipStream_t stream) {
    const char* who = "fm_state_absmax";
    g_err[0] = 0;
    if (count < 0) return fail(FM_ERR_SHAPE, "%s: count %lld < 0", who, (long long)count);
    if (!amax || (count > 0 && !state)) return fail(FM_ERR_NULL, "%s: NULL pointer", who);
    return state_absmax_run(state, count, amax, stream);
}

fm_status fm_mamba2_layer_taps(const fm_layer_desc* d, int64_t batch, int64_t len,
                               fm_layer_taps* taps) {
    g_err[0] = 0;
    if (!taps) return fail(FM_ERR_NULL, "fm_mamba2_layer_taps: taps is NULL");
    fm_status st = check_layer_desc(d, "fm_mamba2_layer_taps");
    if (st != FM_OK) return st;
    layer_taps(d, batch, len, taps);
    return FM_OK;
}


// ---------------------------------------------------------------- outlier-study baselines
size_t fm_quant_per_tensor_workspace_size(void) { return 256; }

fm_status fm_quant_per_tensor(const float* x, int64_t n, int8_t* q, float* scale_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_quant_per_tensor";
    g_err[0] = 0;
    if (!scale_out) return fail(FM_ERR_NULL, "%s: scale_out is NULL", who);
    if (n < 0 || n % 4 || n >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE, "%s: need 0 <= n < 2^31, n a multiple of 4 (n=%lld)", who,
                    (long long)n);
    if (n > 0 && (!x || !q)) return fail(FM_ERR_NULL, "%s: x or q is NULL", who);
    if (n > 0 && (!aligned(x, 16) || !aligned(q, 4)))
        return fail(FM_ERR_SHAPE, "%s: x must be 16-byte and q 4-byte aligned", who);
    fm_status st;
    if ((st = check_ws(workspace, workspace_bytes, fm_quant_per_tensor_workspace_size(), who)) !=
        FM_OK)
        return st;
    return quant_per_tensor_run(x, n, q, scale_out, (float*)workspace, stream);
}

size_t fm_smooth_scales_workspace_size(int64_t k) {
    if (k < 0) return 0;
    return align256((size_t)(2 * k) * sizeof(float));
}

fm_status fm_smooth_scales(const float* x, int64_t rows, const float* w, int64_t n, int64_t k,
                           float* s, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    const char* who = "fm_smooth_scales";
    g_err[0] = 0;
    if (rows < 0 || n < 0 || k <= 0 || rows * k >= ((int64_t)1 << 31) ||
        n * k >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE, "%s: need k > 0, rows, n >= 0, rows*k and n*k < 2^31", who);
    if (!s || (rows > 0 && !x) || (n > 0 && !w)) return fail(FM_ERR_NULL, "%s: NULL argument", who);
    fm_status st;
    if ((st = check_ws(workspace, workspace_bytes, fm_smooth_scales_workspace_size(k), who)) !=
        FM_OK)
        return st;
    return smooth_scales_run(x, rows, w, n, k, s, (float*)workspace, stream);
}

fm_status fm_scale_columns(const float* x, int64_t rows, int64_t k, const float* s,
                           int32_t divide, float* out, hipStream_t stream) {
    const char* who = "fm_scale_columns";
    g_err[0] = 0;
    if (rows < 0 || k <= 0 || rows * k >= ((int64_t)1 << 31))
        return fail(FM_ERR_SHAPE, "%s: need k > 0, rows >= 0, rows*k < 2^31", who);
    if (rows > 0 && (!x || !s || !out)) return fail(FM_ERR_NULL, "%s: NULL argument", who);
    return scale_columns_run(x, rows, k, s, divide, out, stream);
}

fm_status fm_qparams_from_stats(const fm_qparams* st, fm_static_params* out) {
    g_err[0] = 0;
    if (!st || !out) return fail(FM_ERR_NULL, "fm_qparams_from_stats: NULL argument");
    for (int i = 0; i < 2; ++i) {
        const double amax = (double)st->stat_amax[i];
        const double c = amax > 0.0 ? 127.0 / amax : 1.0;
        int e = 0;
        const double m = frexp(c, &e);  // c = m * 2^e, m in [0.5, 1)
        out->sshift[i] = 15 - e;
        out->scoe[i] = (int32_t)nearbyint(ldexp(m, 15));
    }
    // power-of-two points: the same rule as the kernels' pot()
    auto pot_f = [](double a) {
        if (!(a > 0.0)) return 0;
        for (int p = FM_PMAX; p > FM_PMIN; --p)
            if (a * ldexp(1.0, p) <= 127.0) return p;
        return FM_PMIN;
    };
    auto pot_q = [](int64_t m) {
        if (m <= 0) return 0;
        const int64_t lim = (int64_t)127 << 16;
        for (int p = FM_PMAX; p > FM_PMIN; --p) {
            bool ok = p >= 0 ? ((m << p) <= lim) : (m <= (lim << (-p)));
            if (ok) return p;
        }
        return FM_PMIN;
    };
    out->p[0] = pot_f((double)st->stat_amax[2]);
    for (int i = 0; i < 3; ++i) out->p[1 + i] = pot_q(st->stat_amax_q16[i]);
    return FM_OK;
}

}  // extern "C"
