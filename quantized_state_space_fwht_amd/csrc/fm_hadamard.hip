// Hadamard rotation (fast Walsh–Hadamard transform over 256-wide blocks) fused
// with the per-tensor int8 quantization.
//
// Review page of FastMamba, "What carries the argument": Y = (X H)(H^T W^T)
// with H normalized by sqrt(n); referee major comment on Sections III-A / IV-B:
// the scale comes from the maximum of the rotated tensor (Algorithm 1) or is a
// fixed multiply + shift (Fig. 6).
//
// Layout: one wave per 256-block of a row; lane l holds elements 4l..4l+3
// (one 16-byte load).  Butterfly stages h = 1, 2 run inside the lane, stages
// h = 4..128 pair lane l with lane l ^ (h/4).  The stage order is fixed
// (h = 1, 2, ..., 128) because float32 rounding depends on it.
#include "fm_internal.hpp"

namespace fm {

constexpr int kHqThreads = 256;  // 4 waves, one 256-block each per iteration
constexpr int kHqBatch = 4;      // quant pass: blocks per wave whose loads go out together

__device__ __forceinline__ void block_max_to(float m, float* a0, float* a1) {
    __shared__ float red[kHqThreads / 64];
    m = wave_max_f32(m);
    int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) red[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int i = 1; i < kHqThreads / 64; ++i) r = fmaxf(r, red[i]);
        if (a0) atomic_max_nonneg_f32(a0, r);
        if (a1) atomic_max_nonneg_f32(a1, r);
    }
}

// pass 1 (dynamic): grid maximum of |x H| into the slot region (and amax_stats)
__global__ __launch_bounds__(kHqThreads) void hq_amax_kernel(const float* __restrict__ x,
                                                             int64_t nblk_total,
                                                             int32_t* amax_slots,
                                                             float* amax_stats) {
    int lane = threadIdx.x & 63;
    int64_t wv = (int64_t)blockIdx.x * (kHqThreads / 64) + (threadIdx.x >> 6);
    int64_t stride = (int64_t)gridDim.x * (kHqThreads / 64);
    float m = 0.0f;
    int64_t b = wv;
    for (; b + 3 * stride < nblk_total; b += 4 * stride) {  // four blocks' loads in flight
        float4 v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = reinterpret_cast<const float4*>(x + (b + k * stride) * 256)[lane];
#pragma unroll
        for (int k = 0; k < 4; ++k) m = fmaxf(m, absmax4(fwht256_lane(v[k], lane)));
    }
    for (; b < nblk_total; b += stride) {
        float4 v = reinterpret_cast<const float4*>(x + b * 256)[lane];
        m = fmaxf(m, absmax4(fwht256_lane(v, lane)));
    }
    __shared__ float red[kHqThreads / 64];
    m = wave_max_f32(m);
    if (lane == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int i = 1; i < kHqThreads / 64; ++i) r = fmaxf(r, red[i]);
        slot_max(amax_slots, blockIdx.x, (int32_t)__float_as_uint(r));
        if (amax_stats) atomic_max_nonneg_f32(amax_stats, r);
    }
}

__device__ __forceinline__ float scale_coef(fm_scale_mode mode, int32_t scoe, int32_t sshift,
                                            float amax) {
    if (mode == FM_SCALE_DYNAMIC) return amax == 0.0f ? 1.0f : 127.0f / amax;
    return ldexpf((float)scoe, -sshift);
}

// pass 2 (or the only pass in static mode): rotate again and quantize
// amax_slots (dynamic, nullable): the grid maximum is the slot region's, and
// block 0 also stores it to amax_ws; otherwise it is read from amax_ws.
__global__ __launch_bounds__(kHqThreads) void hq_quant_kernel(
    const float* __restrict__ x, int64_t nblk_total, fm_scale_mode mode, int32_t scoe,
    int32_t sshift, float* amax_ws, const int32_t* amax_slots, char4* __restrict__ q,
    float* scale_out, float* amax_stats, int rotated_input, fm_quant_stats* qs, int qpt) {
    int lane = threadIdx.x & 63;
    int64_t wv = (int64_t)blockIdx.x * (kHqThreads / 64) + (threadIdx.x >> 6);
    int64_t stride = (int64_t)gridDim.x * (kHqThreads / 64);
    // the first block's load goes out before the scale is known
    float4 v0 = wv < nblk_total ? reinterpret_cast<const float4*>(x + wv * 256)[lane]
                                : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    float amax = 0.0f;
    if (mode == FM_SCALE_DYNAMIC) {
        if (amax_slots) {  // wave 0 reduces the slots, LDS shares
            __shared__ float amax_s;
            if (threadIdx.x < 64) {
                const float v = __int_as_float(slots_wave_max(amax_slots));
                if (threadIdx.x == 0) amax_s = v;
            }
            __syncthreads();
            amax = amax_s;
        } else {
            amax = *amax_ws;
        }
    }
    float c = scale_coef(mode, scoe, sshift, amax);
    const float s_dq = 1.0f / c;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *scale_out = s_dq;
        if (amax_slots) *amax_ws = amax;
    }
    float m = 0.0f;
    QStat st;
    // kHqBatch blocks per wave and round, their loads issued together
    for (int64_t b0 = wv; b0 < nblk_total; b0 += kHqBatch * stride) {
        float4 vb[kHqBatch];
#pragma unroll
        for (int k = 0; k < kHqBatch; ++k) {
            const int64_t b = b0 + k * stride;
            vb[k] = (b0 == wv && k == 0) ? v0
                    : (b < nblk_total ? reinterpret_cast<const float4*>(x + b * 256)[lane]
                                      : make_float4(0.0f, 0.0f, 0.0f, 0.0f));
        }
#pragma unroll
        for (int k = 0; k < kHqBatch; ++k) {
            const int64_t b = b0 + k * stride;
            if (b >= nblk_total) break;
            float4 v = vb[k];
            if (!rotated_input) v = fwht256_lane(v, lane);
            m = fmaxf(m, absmax4(v));
            q[b * 64 + lane] = quant4(v, c);
            if (qs) quant_stat4(st, v, c, s_dq);
        }
    }
    if (qs) qstat_flush(st, qs, qpt);
    if (amax_stats) block_max_to(m, amax_stats, nullptr);
}

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

static int hq_grid(int64_t nblk_total, int64_t cap = 4096) {
    int64_t g = (nblk_total + 3) / 4;
    if (g > cap) g = cap;
    return (int)(g < 1 ? 1 : g);
}

fm_status zero_words(void* p, int64_t n, hipStream_t s) {
    if (n <= 0) return FM_OK;
    int g = (int)((n + 255) / 256);
    if (g > 1024) g = 1024;
    zero_words_kernel<<<g, 256, 0, s>>>((uint32_t*)p, n);
    return check_launch("zero_words");
}

fm_status hq_run(const float* x, int64_t rows, int64_t k, fm_scale_mode mode, int32_t scoe,
                 int32_t sshift, int8_t* q, float* scale_out, float* amax_stats, float* amax_ws,
                 int32_t* amax_slots, hipStream_t s, fm_quant_stats* qs, int qpt) {
    int64_t nb = rows * (k / 256);
    int g = hq_grid((nb + kHqBatch - 1) / kHqBatch);
    fm_status st;
    if (mode == FM_SCALE_DYNAMIC) {  // amax_slots must hold 0 (zeroed by the caller)
        // few workgroups (grid-stride): four blocks per wave at least (their loads
        // go out together), one slot atomic per workgroup
        hq_amax_kernel<<<hq_grid((nb + 3) / 4, 512), kHqThreads, 0, s>>>(x, nb, amax_slots,
                                                                         amax_stats);
        if ((st = check_launch("hq_amax_kernel")) != FM_OK) return st;
        hq_quant_kernel<<<g, kHqThreads, 0, s>>>(x, nb, mode, scoe, sshift, amax_ws, amax_slots,
                                                 (char4*)q, scale_out, nullptr, 0, qs, qpt);
    } else {
        hq_quant_kernel<<<g, kHqThreads, 0, s>>>(x, nb, mode, scoe, sshift, nullptr, nullptr,
                                                 (char4*)q, scale_out, amax_stats, 0, qs, qpt);
    }
    return check_launch("hq_quant_kernel");
}

// ---------------------------------------------------------------- pre-norm + rotation
// A stack feeds each layer RMSNorm(h) (weight 1; the fixed summation order of
// the gate's RMSNorm: 64 lane-strided partial sums in ascending order, then the
// xor butterfly), rotated and quantized like any in_proj input.  Fused here so
// the normalized rows never go to memory: a workgroup takes kNormRows rows,
// two waves each; a row is staged in LDS, its first wave forms
// r = 1 / sqrt(ss / d + 1e-5) (or reads the r that pass 1 stored), and the
// row's two waves rotate its 256-blocks of (h_i * r) * 1.  Two rows per
// workgroup keep twice the bytes in flight per CU for the same wave count.
// Dynamic mode: pass 1 takes the rotated maximum into a slot region and stores
// r per row; pass 2 reads h again and writes the codes (9 bytes per element in
// all, against 17 for a separate normalization followed by the two passes).
// Static mode: one pass.
constexpr int kNormRows = 2;
constexpr int kNormWaves = 2;  // per row
constexpr int kNormThreads = 64 * kNormWaves * kNormRows;

template <bool kQuant>
__global__ __launch_bounds__(kNormThreads) void norm_hq_kernel(
    const float* __restrict__ h, int64_t rows, int dm, float* __restrict__ rs, fm_scale_mode mode,
    int32_t scoe, int32_t sshift, float* amax_ws, int32_t* amax_slots, char4* __restrict__ q,
    float* scale_out, float* amax_stats, fm_quant_stats* qs, int qpt) {
    extern __shared__ __attribute__((aligned(16))) float rows_buf[];  // kNormRows x dm floats
    __shared__ float r_s[kNormRows], c_s, wmax[kNormThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int sub = wave / kNormWaves, wv = wave % kNormWaves;  // row of the workgroup, wave in it
    const int st = tid % (64 * kNormWaves);                     // thread within the row's waves
    const int64_t r0 = blockIdx.x * (int64_t)kNormRows + sub;
    const bool live = r0 < rows;  // the last workgroup's second row may lie past the end
    float* row = rows_buf + sub * dm;
    const float* hr = h + (live ? r0 : rows - 1) * dm;
    constexpr int kRowThreads = 64 * kNormWaves;
    constexpr int kLd = 8;  // loads in flight per thread: rows up to 4096 floats in one round
    for (int i0 = st * 4; i0 < dm; i0 += 4 * kLd * kRowThreads) {
        float4 v[kLd];
#pragma unroll
        for (int k = 0; k < kLd; ++k) {
            const int i = i0 + k * 4 * kRowThreads;
            v[k] = i < dm ? *reinterpret_cast<const float4*>(hr + i) : make_float4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < kLd; ++k) {
            const int i = i0 + k * 4 * kRowThreads;
            if (i < dm) *reinterpret_cast<float4*>(row + i) = v[k];
        }
    }
    const bool have_r = kQuant && mode == FM_SCALE_DYNAMIC;  // pass 2 reads pass 1's r
    __syncthreads();
    if (wv == 0) {
        float r;
        if (have_r) {
            r = live ? rs[r0] : 1.0f;
        } else {
            // ascending i within this lane (the fixed order): groups of 16 steps
            // of 64 whose reads go out together, then the rest in groups of 4
            // (dm % 256 == 0)
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
            r = 1.0f / sqrtf(ss / (float)dm + 1e-5f);
            if (!kQuant && live && lane == 0) rs[r0] = r;
        }
        if (lane == 0) r_s[sub] = r;
    }
    if constexpr (kQuant) {
        if (wave == 0) {
            float amax = 0.0f;
            if (mode == FM_SCALE_DYNAMIC) amax = __int_as_float(slots_wave_max(amax_slots));
            const float c = mode == FM_SCALE_DYNAMIC ? (amax == 0.0f ? 1.0f : 127.0f / amax)
                                                     : ldexpf((float)scoe, -sshift);
            if (lane == 0) {
                c_s = c;
                if (blockIdx.x == 0) {
                    *scale_out = 1.0f / c;
                    if (mode == FM_SCALE_DYNAMIC) *amax_ws = amax;
                }
            }
        }
    }
    __syncthreads();
    const float r = r_s[sub], c = kQuant ? c_s : 0.0f, s_dq = kQuant ? 1.0f / c : 0.0f;
    float m = 0.0f;
    QStat stt;
    for (int blk = wv; live && blk < dm / 256; blk += kNormWaves) {
        float4 v = *reinterpret_cast<const float4*>(row + blk * 256 + lane * 4);
        v.x = (v.x * r) * 1.0f;
        v.y = (v.y * r) * 1.0f;
        v.z = (v.z * r) * 1.0f;
        v.w = (v.w * r) * 1.0f;
        v = fwht256_lane(v, lane);
        m = fmaxf(m, absmax4(v));
        if constexpr (kQuant) {
            q[(r0 * dm + blk * 256) / 4 + lane] = quant4(v, c);
            if (qs) quant_stat4(stt, v, c, s_dq);
        }
    }
    if (kQuant && qs) qstat_flush(stt, qs, qpt);
    if (!kQuant || amax_stats) {
        m = wave_max_f32(m);
        if (lane == 0) wmax[wave] = m;
        __syncthreads();
        if (tid == 0) {
            // rows past the end contribute 0; maxima are exact in any order
            for (int k = 1; k < kNormThreads / 64; ++k) m = fmaxf(m, wmax[k]);
            if constexpr (!kQuant) slot_max(amax_slots, blockIdx.x, (int32_t)__float_as_uint(m));
            else atomic_max_nonneg_f32(amax_stats, m);
        }
    }
}

fm_status norm_hq_run(const float* h, int64_t rows, int64_t dm, fm_scale_mode mode, int32_t scoe,
                      int32_t sshift, int8_t* q, float* scale_out, float* amax_stats,
                      float* amax_ws, int32_t* amax_slots, float* rs, hipStream_t s,
                      fm_quant_stats* qs, int qpt) {
    if (rows == 0) return FM_OK;
    const size_t lds = (size_t)kNormRows * dm * sizeof(float);
    const unsigned grid = (unsigned)((rows + kNormRows - 1) / kNormRows);
    fm_status st;
    if (mode == FM_SCALE_DYNAMIC) {  // amax_slots must hold 0 (zeroed by the caller)
        norm_hq_kernel<false><<<grid, kNormThreads, lds, s>>>(
            h, rows, (int)dm, rs, mode, scoe, sshift, amax_ws, amax_slots, nullptr, nullptr,
            nullptr, nullptr, qpt);
        if ((st = check_launch("norm_hq_kernel(max)")) != FM_OK) return st;
    }
    norm_hq_kernel<true><<<grid, kNormThreads, lds, s>>>(
        h, rows, (int)dm, mode == FM_SCALE_DYNAMIC ? rs : nullptr, mode, scoe, sshift, amax_ws,
        amax_slots, (char4*)q, scale_out, amax_stats, qs, qpt);
    return check_launch("norm_hq_kernel(codes)");
}

fm_status hq_quant_rotated(const float* r, int64_t rows, int64_t k, fm_scale_mode mode,
                           int32_t scoe, int32_t sshift, float* amax_ws,
                           const int32_t* amax_slots, int8_t* q, float* scale_out,
                           hipStream_t s, fm_quant_stats* qs, int qpt) {
    int64_t nb = rows * (k / 256);
    hq_quant_kernel<<<hq_grid((nb + kHqBatch - 1) / kHqBatch), kHqThreads, 0, s>>>(
                                                       r, nb, mode, scoe, sshift, amax_ws,
                                                       amax_slots, (char4*)q, scale_out, nullptr,
                                                       1, qs, qpt);
    return check_launch("hq_quant_kernel(rotated)");
}

}  // namespace fm
