// Internal host-side declarations shared by the library's translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fm.h"
#include "fm_device.hpp"

namespace fm {

// ---------------------------------------------------------------- errors
void set_error(const char* fmt, ...);
fm_status fail(fm_status s, const char* fmt, ...);
// hipGetLastError after a launch; FM_ERR_HIP with the kernel name on failure
fm_status check_launch(const char* what);

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Bump allocator over a caller workspace.  With a null base it only measures:
// the returned "pointers" are then byte offsets from the start of the workspace.
struct Arena {
    uintptr_t base;
    size_t used;
    explicit Arena(void* b) : base((uintptr_t)b), used(0) {}
    template <class T>
    T* take(size_t count) {
        T* p = (T*)(base + used);
        used += align256(count * sizeof(T));
        return p;
    }
};

// ---------------------------------------------------------------- layer scalars
// Small per-call block at the head of a layer workspace (32-bit words).  The
// dynamic scales and exponents flow from kernel to kernel through it and are
// never copied to the host.
enum SmallSlot {
    kAmaxU = 0,     // float: max |u H|
    kAmaxG = 1,     // float: max |n H|
    kAmaxXbc = 2,   // float: max |xBC|
    kAmaxQ = 3,     // int[3]: max |x|, |B|, |C| in Q.16
    kScaleU = 6,    // float: in_proj input dequant scale
    kScaleG = 7,    // float: out_proj input dequant scale
    kP = 8,         // int[4]: p_c, p_x, p_B, p_C
    kSmallWords = 16
};
// Slot regions of a layer workspace (slotted grid maxima, fm_device.hpp)
enum SlotRegion {
    kRegionConvX = 0,  // conv pass: max |SiLU| of x, B, C in Q.16 (three regions)
    kRegionG = 3,      // gate pass: max |n H| as float bits
    kRegionXbc = 4,    // in_proj epilogue: max |xBC| as float bits
    kRegionU = 5,      // in_proj input rotation: max |u H| as float bits
    kRegions = 6
};

// Publish what a layer call used into qp (scales, exponents, statistics) and,
// when given, the exponents into the cache.  One thread, after every kernel
// that writes the block has completed.
__device__ inline void layer_publish(const uint32_t* small, fm_qparams* qp, int32_t* cache_p) {
    uint32_t v[kP + 4];  // every load before the first store: one round trip
#pragma unroll
    for (int k = 0; k < kP + 4; ++k) v[k] = small[k];
    qp->scale[0] = __uint_as_float(v[kScaleU]);
    qp->scale[1] = __uint_as_float(v[kScaleG]);
#pragma unroll
    for (int k = 0; k < 4; ++k) qp->p[k] = (int32_t)v[kP + k];
    if (cache_p)
#pragma unroll
        for (int k = 0; k < 4; ++k) cache_p[k] = (int32_t)v[kP + k];
    atomicMax((unsigned int*)&qp->stat_amax[0], v[kAmaxU]);
    atomicMax((unsigned int*)&qp->stat_amax[1], v[kAmaxG]);
    atomicMax((unsigned int*)&qp->stat_amax[2], v[kAmaxXbc]);
#pragma unroll
    for (int k = 0; k < 3; ++k) atomicMax(&qp->stat_amax_q16[k], (int32_t)v[kAmaxQ + k]);
}

// ---------------------------------------------------------------- launchers
// Zero `n` 32-bit words (a kernel, so it can sit inside captured graphs).
fm_status zero_words(void* p, int64_t n, hipStream_t s);

// Hadamard rotation + per-tensor int8.  In dynamic mode the first pass leaves
// the grid maximum in the slot region `amax_slots` (zeroed by the caller) and
// the second writes it to `amax_ws` (one float).
// qs (nullable): quantization statistics of point qpt (fm_quant_stats)
fm_status hq_run(const float* x, int64_t rows, int64_t k, fm_scale_mode mode, int32_t scoe,
                 int32_t sshift, int8_t* q, float* scale_out, float* amax_stats, float* amax_ws,
                 int32_t* amax_slots, hipStream_t s, fm_quant_stats* qs = nullptr, int qpt = 0);
// second pass only: quantize already-rotated rows r (dynamic: amax_ws holds the max)
// amax_slots (dynamic): the slot region holding the grid maximum; it is also
// written to amax_ws
fm_status hq_quant_rotated(const float* r, int64_t rows, int64_t k, fm_scale_mode mode,
                           int32_t scoe, int32_t sshift, float* amax_ws,
                           const int32_t* amax_slots, int8_t* q, float* scale_out,
                           hipStream_t s, fm_quant_stats* qs = nullptr, int qpt = 0);

struct GemmEpilogue {
    int32_t* acc = nullptr;
    int64_t ld_acc = 0;
    float* out = nullptr;
    int64_t ld_out = 0;
    const float* s_a = nullptr;
    const float* s_b = nullptr;
    const float* resid = nullptr;  // out = resid + acc * s (pre-norm residual stacks)
    int64_t ld_resid = 0;
    float* amax = nullptr;         // max |out| over columns [amax_c0, amax_c1)
    int32_t* amax_slots = nullptr; // instead of amax (tiled and plain few-rows kernels): a
                                   // slot region receiving that maximum as float bits
    int64_t amax_c0 = 0, amax_c1 = 0;
    // one-token step (few-rows kernel only): the columns [amax_c0, amax_c1) are
    // xBC and go through its power-of-two quantization, the conv window held in
    // conv_state, SiLU and the requantization to x / B / C codes
    const int8_t* conv_w_q = nullptr;   // [ch, 4]
    const int32_t* conv_p_w = nullptr;  // [ch]
    const int32_t* conv_b_q16 = nullptr;
    const int32_t* conv_p = nullptr;    // device int32[4]: p_c, p_x, p_B, p_C
    int8_t* conv_state = nullptr;       // [rows, ch, 3] in/out
    int8_t* x_out = nullptr;            // [rows, d_inner]
    int8_t* b_out = nullptr;            // [rows, dstate]
    int8_t* c_out = nullptr;
    int8_t* xbc_q = nullptr;            // nullable: [rows, ch] quantized conv input
    int32_t* conv_amax_slots = nullptr; // three slot regions: max |SiLU| of x, B, C (Q.16);
                                        // max |xBC| goes to amax_slots
    int64_t d_inner = 0, dstate = 0;
    float* sz_out = nullptr;            // [rows, d_inner]: SiLU(z) of the z columns [0, amax_c0)
    // dt columns [amax_c1, n): also dt = SoftPlus(dt_in) and dA = e^(dt * A) in Q.16
    // (row-major [rows, n - amax_c1]), for the one-step scan
    const float* dt_bias = nullptr;
    const int32_t* a_q16 = nullptr;
    int32_t* dt_out = nullptr;
    int32_t* da_out = nullptr;
    bool write_xbc = false;             // also write the float z and xBC columns to out
    // one-token step (few-rows kernel only): A comes as rotated float rows with
    // their row maxima; every workgroup forms the tensor scale c from them
    // (dynamic: 127 / max, static: scoe * 2^-sshift) and quantizes its A slices
    // while loading them, so no pass over A separates the row kernel from the
    // product.  Workgroup 0 stores the maximum, the dequant scale 1 / c and,
    // when a_q_tap is set, the codes.
    const float* a_f = nullptr;         // [m, k] rotated rows
    const float* a_rowmax = nullptr;    // [m] max |row|
    fm_scale_mode a_mode = FM_SCALE_DYNAMIC;
    int32_t a_scoe = 0, a_sshift = 0;
    float* a_amax_out = nullptr;
    float* a_scale_out = nullptr;
    int8_t* a_q_tap = nullptr;
    // after the product: one thread publishes the layer's block (layer_publish)
    const uint32_t* pub_small = nullptr;
    fm_qparams* pub_qp = nullptr;
    int32_t* pub_cache_p = nullptr;
};
// int8 codes of m <= 64 rotated rows (x [m, k] float, 16-byte aligned) with the
// tensor scale from their row maxima; writes the dequant scale and the maximum
fm_status quant_rows_run(const float* x, const float* rowmax, int64_t m, int64_t k,
                         fm_scale_mode mode, int32_t scoe, int32_t sshift, int8_t* q,
                         float* scale_out, float* amax_out, hipStream_t s);
fm_status gemm_run(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k,
                   const GemmEpilogue& ep, hipStream_t s);

// conv: quantize xBC, conv, SiLU.  Dynamic: hands the SiLU values to the requant
// pass through s16 and the part maxima through slot regions (the requant pass
// writes amax_q16[3] and the codes); static (p given): writes codes directly.
struct ConvArgs {
    const float* xbc;
    int64_t xbc_stride;
    int64_t batch, len, d_inner, dstate;
    const int8_t* w_q;
    const int32_t* p_w;
    const int32_t* b_q16;
    float* xbc_amax;           // dynamic: max |xBC| (written by workgroup 0 from the slots)
    const int32_t* xbc_amax_slots;  // dynamic: slot region of max |xBC| (GEMM epilogue or a pass)
    const int32_t* p_fixed;    // static: device int32[4]
    const int8_t* state_in;
    int8_t* state_out;
    int8_t* xbc_q;
    int32_t* s16;              // dynamic: [T, ch] SiLU outputs between the passes (Q.16, or
                               // 16-bit words at per-wave exponents and their table)
    int32_t* amax_q16;         // dynamic: [3] the part maxima (written by the requant pass)
    int32_t* amax_slots;       // dynamic: three slot regions (x, B, C) zeroed before
    int8_t* x_out;
    int8_t* b_out;
    int8_t* c_out;
    int32_t* p_out;            // [4]
    int32_t* amax_stats;       // nullable [4]
    // nullable: extra workgroups also form dt and the decay of every (token, head)
    // (the scan's prologue) from the in_proj dt columns
    const float* dt_raw;
    int64_t dt_stride;
    const float* dt_bias;
    const int32_t* a_q16;
    int64_t nheads;
    int32_t* dt_out;           // [T, H]
    int32_t* da_out;
    fm_quant_stats* qs;        // nullable: statistics of the xBC, x, B, C points
};
fm_status conv_run(const ConvArgs& a, hipStream_t s);
// max |x| of a strided matrix into a slot region (zeroed before)
fm_status amax_strided_run(const float* x, int64_t rows, int64_t cols, int64_t stride,
                           int32_t* amax_slots, hipStream_t s);

struct ScanArgs {
    const int8_t* x;
    const int8_t* bm;
    const int8_t* cm;
    const float* dt_raw;
    int64_t dt_stride;
    const float* dt_bias;
    const int32_t* a_q16;
    const int32_t* d_q16;
    const int32_t* p;
    int64_t batch, len, nheads, headdim, dstate;
    const int32_t* state_in;
    int32_t* state_out;
    int32_t* y;
    int32_t* dt_out;           // [T, H] written by the dt / decay prologue (required)
    int32_t* da_out;
    bool dt_ready;             // dt_out / da_out already hold them: no prologue launch
    // One-step scans only: state_in / state_out hold codes of state_bits bits
    // (16: int16; 24: three little-endian bytes) on the grid 2^state_shift of
    // the state's own, behind the int32 pointer type.  0 or 32: int32 values.
    int state_bits;
    int state_shift;
};
// dt and the decay of every (token, head) into dt_out / da_out
fm_status scan_prep_run(const ScanArgs& a, hipStream_t s);
// chunked (SSD-form) variant: the recurrence without per-step rounding, in
// float64 over chunks of kSsdChunk tokens (fm_ssd.hip); headdim 64 only
constexpr int kSsdChunk = 64;
size_t ssd_ws_bytes(int64_t batch, int64_t len, int64_t nheads, int64_t headdim, int64_t dstate);
fm_status ssd_run(const ScanArgs& a, void* ws, hipStream_t s, hipEvent_t ev_start = nullptr,
                  hipEvent_t ev_stop = nullptr);
// workspace of the scan (none: B and C are staged through LDS)
size_t scan_ws_bytes(int64_t batch, int64_t len, int64_t dstate);
// ev_start / ev_stop (nullable): recorded on s right around the scan kernel
fm_status scan_run(const ScanArgs& a, void* ws, hipStream_t s, hipEvent_t ev_start = nullptr,
                   hipEvent_t ev_stop = nullptr);

struct GateArgs {
    const int32_t* y;
    const float* z;
    int64_t z_stride;
    const int32_t* p;
    const float* norm_w;
    int64_t rows, d_inner;
    fm_scale_mode mode;
    int32_t scoe, sshift;
    int8_t* q;
    float* scale_out;
    float* amax_stats;
    float* normed_out;
    float* rot_ws;     // dynamic: [rows, d_inner] rotated values between passes
    float* amax_ws;    // dynamic: 1 float, the grid maximum (written by the quant pass)
    int32_t* amax_slots;  // dynamic: a slot region zeroed before (the gate pass's maxima)
    const float* sz;   // nullable: SiLU(z) already formed ([rows, d_inner], Q.16 as float)
    fm_quant_stats* qs;  // nullable: statistics of the out_proj input point
    float* rowmax;     // nullable: one-token form, rotated rows to rot_ws and their maxima
                       // here (the out_proj product quantizes them); q, scale_out unused
    // one-token form: workgroup 0 also reduces the in_proj epilogue's slotted
    // maxima (max |xBC|, max |SiLU| of x, B, C) into the call's small block
    const int32_t* step_slots;
    uint32_t* step_small;
};
fm_status gate_run(const GateArgs& a, hipStream_t s);

// knots: nullable host array of nine Q.30 values replacing the chord table
fm_status nau_run(int fn, const int32_t* x, int32_t* y, int64_t n, hipStream_t s,
                  const int64_t* knots = nullptr);

// outlier-study baselines (fm_outlier.hip); n a multiple of 4, ws as documented in fm.h
fm_status quant_per_tensor_run(const float* x, int64_t n, int8_t* q, float* scale_out,
                               float* amax_ws, hipStream_t s);
fm_status smooth_scales_run(const float* x, int64_t rows, const float* w, int64_t n, int64_t k,
                            float* s_out, float* ws, hipStream_t s);
fm_status scale_columns_run(const float* x, int64_t rows, int64_t k, const float* sc, int divide,
                            float* out, hipStream_t s);

// layer pipeline (fm_layer.hip)
size_t layer_ws_bytes(const fm_layer_desc* d, int64_t batch, int64_t len);
void layer_taps(const fm_layer_desc* d, int64_t batch, int64_t len, fm_layer_taps* t);
// compute units of the current device (queried once per device)
int device_cus();

// the per-call options of a layer call (fm_layer_opts, validated)
struct LayerOpts {
    bool keep = false;               // also write the intermediates the taps name
    fm_quant_stats* qs = nullptr;    // prefill: add the quantization statistics here
    hipEvent_t ev[FM_LAYER_EVENTS] = {};  // stage boundaries (fm_layer_opts.stage_events)
};
// state_bits / state_shift: the decode cache's state format (ScanArgs);
// ssd_ws (prefill only): run the chunked scan variant with this workspace
fm_status layer_run(const fm_layer_desc* d, const fm_layer_weights* W, const fm_static_params* sp,
                    const float* u, int64_t batch, int64_t len, float* out, const fm_cache* cache,
                    fm_qparams* qp, void* workspace, bool decode, hipStream_t s,
                    const LayerOpts& opts, int state_bits = 32, int state_shift = 0,
                    void* ssd_ws = nullptr);

// narrow state codes (fm_state.hip)
fm_status state_narrow_run(const int32_t* h, int64_t n, int bits, int shift, void* out,
                           hipStream_t s);
fm_status state_widen_run(const void* c, int64_t n, int bits, int shift, int32_t* out,
                          hipStream_t s);
fm_status state_absmax_run(const int32_t* h, int64_t n, uint32_t* amax, hipStream_t s);
fm_status prepare_run(const fm_layer_desc* d, const float* w_in, const float* w_out,
                      const float* conv_w, const float* conv_b, const float* a, const float* dv,
                      int8_t* w_in_q, float* s_w_in, int8_t* w_out_q, float* s_w_out,
                      int8_t* conv_w_q, int32_t* conv_p_w, int32_t* conv_b_q16, int32_t* a_q16,
                      int32_t* d_q16, void* ws, hipStream_t s);

// pre-norm of the residual stream fused with the in_proj input rotation and
// quantization (hq_run's arguments; rs: [rows] floats of scratch for 1/rms)
fm_status norm_hq_run(const float* h, int64_t rows, int64_t dm, fm_scale_mode mode, int32_t scoe,
                      int32_t sshift, int8_t* q, float* scale_out, float* amax_stats,
                      float* amax_ws, int32_t* amax_slots, float* rs, hipStream_t s,
                      fm_quant_stats* qs, int qpt);

}  // namespace fm
