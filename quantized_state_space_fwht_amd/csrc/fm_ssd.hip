// Chunked (SSD-form) prefill scan: a separate, faster variant of the
// fixed-point scan.  The sequential scan rounds the state onto its grid at
// every step; summed over chunks of tokens in matrix form (Mamba2's state
// space duality, a sequence-chunked schedule), the recurrence can only be
// computed without that rounding.  This variant computes, in float64 and in
// the state's own grid units,
//     h_t = a_t h_{t-1} + dt_t x_t[p] B_t[n] / 2^8,   a_t = dA_t / 2^16
//     y_t = sat32(floor(sum_n C_t[n] h_t / 2^(p_B + p_C) + 1/2) + rshr(D x_t, 8))
// and rounds the final state onto the grid; it does not saturate inside the
// sequence.  Contract: y within one step of the correctly rounded real
// recurrence (float64 summation order only), and within the propagated
// half-step bound of the sequential scan, plus one step.
//
// Three kernels per call, chunk = 64 tokens, headdim 64 (the contractions on
// the float64 and int8 matrix cores):
//  ssd_chunk_state_kernel  (chunk, head, batch): the chunk's own state
//      S_c = sum_s w_s x_s (x) B_s, w_s = dt_s / 2^8 * prod_{s<r<end} a_r, and
//      its total decay A_c; S_c to the workspace.
//  ssd_chunk_scan_kernel   one thread per state element: H_in(c) = the state
//      entering chunk c (overwrites S_c), H <- A_c H + S_c over the chunks; the
//      final state rounded to the grid.
//  ssd_chunk_out_kernel    (chunk, head, batch): G = C B^T of the chunk (int8
//      dot products, exact), M[t,s] = G[t,s] prod_{s<r<=t} a_r dt_s / 2^8 for
//      s <= t; y_acc = M x + (prod_{r<=t} a_r) C H_in^T; y rounded as above.
// Work per (chunk, head): about 0.5 M + 0.5 M + 0.25 M float64 multiply-adds
// (d_state 128); the variant is bound by the float64 rate, not by HBM.
#include "fm_internal.hpp"

namespace fm {

namespace {
constexpr int Q = kSsdChunk;  // tokens per chunk
constexpr int kSsdP = 64;        // headdim
}  // namespace

size_t ssd_ws_bytes(int64_t batch, int64_t len, int64_t nheads, int64_t headdim, int64_t dstate) {
    const int64_t nc = (len + Q - 1) / Q;
    return align256((size_t)(batch * nheads * nc * headdim * dstate) * sizeof(double)) +
           align256((size_t)(batch * nheads * nc) * sizeof(double));
}

// ------------------------------------------------------------------ matrix cores
typedef double f64x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// D (16 x 16) += A (16 x 4) B (4 x 16) in float64.  Lane l holds A[l % 16][l / 16]
// and B[l / 16][l % 16]; element v of D is D[l / 16 + 4 v][l % 16] (rows
// interleaved, unlike the int8 form below).
__device__ __forceinline__ f64x4 mfma_f64(double a, double b, f64x4 c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

// D (16 x 16) += A (16 x 32) B (32 x 16) over int8 codes, exact in int32.  Lane l
// holds A[l % 16][8 (l / 16) .. + 7] and B[8 (l / 16) .. + 7][l % 16] as 8 packed
// bytes; element v of D is D[4 (l / 16) + v][l % 16].
__device__ __forceinline__ i32x4 mfma_i8(int64_t a, int64_t b, i32x4 c) {
    return __builtin_amdgcn_mfma_i32_16x16x32_i8(a, b, c, 0, 0, 0);
}

// 64-lane products over lanes: lane l holds v_l.  Inclusive prefix
// prod_{r<=l} v_r and inclusive suffix prod_{r>=l} v_r, in six shuffle steps.
__device__ __forceinline__ double wave_prefix_prod(double v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double u = __shfl_up(v, off, 64);
        if (lane >= off) v *= u;
    }
    return v;
}
__device__ __forceinline__ double wave_prefix_sum(double v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double u = __shfl_up(v, off, 64);
        if (lane >= off) v += u;
    }
    return v;
}
__device__ __forceinline__ double wave_suffix_prod(double v, int lane) {
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const double u = __shfl_down(v, off, 64);
        if (lane + off < 64) v *= u;
    }
    return v;
}

// ------------------------------------------------------------------ chunk states
// The chunk's own state, stored transposed: S^T[n][p] = sum_s B[s][n] (w_s x[s][p])
// with w_s = dt_s / 2^8 * prod_{s<r<Q} a_r, on the float64 matrix cores; wave w
// owns the n tiles w * NTW .. w * NTW + NTW - 1 and every p (4 tiles).
template <int N>
__global__ __launch_bounds__(256) void ssd_chunk_state_kernel(ScanArgs A, double* __restrict__ S,
                                                              double* __restrict__ Ad, int nc) {
    __shared__ double w_s[Q];
    __shared__ double xw[Q][kSsdP + 1];  // x[s][p] (scaled by w_s as it is read)
    __shared__ __attribute__((aligned(16))) int8_t bs[Q][N];  // B codes
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = (int)A.nheads;
    const int64_t L = A.len;
    const int t0 = c * Q;
    const int q = (int)(L - t0 < Q ? L - t0 : Q);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    // staging: every global load of a thread issued before any LDS store
    double av = 1.0, dv = 0.0;  // wave 0: a and dt / 2^8 of token `lane` (padding 1, 0)
    if (wave == 0 && lane < q) {
        const int64_t i = ((int64_t)b * L + t0 + lane) * H + h;
        av = (double)A.da_out[i] * 0x1p-16;
        dv = (double)A.dt_out[i] * 0x1p-8;
    }
    {
        const int xr = tid >> 2, xc = 16 * (tid & 3);  // x: 64 rows of 64 bytes
        int4 xv = {0, 0, 0, 0};
        if (xr < q)
            xv = *reinterpret_cast<const int4*>(A.x + (((int64_t)b * L + t0 + xr) * H + h) * kSsdP + xc);
        constexpr int BL = Q * N / 16 / 256;  // B: 16-byte pieces per thread
        int4 bv[BL];
#pragma unroll
        for (int k = 0; k < BL; ++k) {
            const int e = tid + 256 * k, br = e / (N / 16), bc = 16 * (e % (N / 16));
            bv[k] = br < q ? *reinterpret_cast<const int4*>(A.bm + ((int64_t)b * L + t0 + br) * N + bc)
                           : int4{0, 0, 0, 0};
        }
        const int8_t* xb = reinterpret_cast<const int8_t*>(&xv);
#pragma unroll
        for (int k = 0; k < 16; ++k) xw[xr][xc + k] = (double)xb[k];
#pragma unroll
        for (int k = 0; k < BL; ++k) {
            const int e = tid + 256 * k, br = e / (N / 16), bc = 16 * (e % (N / 16));
            *reinterpret_cast<int4*>(&bs[br][bc]) = bv[k];
        }
    }
    if (wave == 0) {  // w_s = dt_s / 2^8 * prod_{s<r<Q} a_r; A_c = prod of all
        const double suf = wave_suffix_prod(av, lane);   // prod_{r>=lane}
        const double after = __shfl_down(suf, 1, 64);     // prod_{r>lane}
        w_s[lane] = dv * (lane == 63 ? 1.0 : after);
        if (lane == 0) Ad[((int64_t)b * H + h) * nc + c] = suf;
    }
    __syncthreads();
    constexpr int NTW = N / 64;  // n tiles per wave
    f64x4 acc[NTW][4];
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};
    for (int s0 = 0; s0 < Q; s0 += 4) {
        double bx[4];
        const double ws = w_s[s0 + lk];
#pragma unroll
        for (int j = 0; j < 4; ++j) bx[j] = xw[s0 + lk][16 * j + lr] * ws;
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
            const double ab = (double)bs[s0 + lk][16 * (NTW * wave + i) + lr];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = mfma_f64(ab, bx[j], acc[i][j]);
        }
    }
    double* Sc = S + (((int64_t)b * H + h) * nc + c) * (int64_t)(kSsdP * N);
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                Sc[(16 * (NTW * wave + i) + lk + 4 * v) * kSsdP + 16 * j + lr] = acc[i][j][v];
}

// ------------------------------------------------------------------ across chunks
// One thread per state element, in the workspace's [n][p] order per chunk.
__global__ __launch_bounds__(256) void ssd_chunk_scan_kernel(ScanArgs A, double* __restrict__ S,
                                                             const double* __restrict__ Ad, int nc,
                                                             int64_t pn_count) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (b, h, n, p)
    if (e >= A.batch * A.nheads * pn_count) return;
    const int64_t bh = e / pn_count, np = e - bh * pn_count;
    const int64_t n = np / kSsdP, p = np - n * kSsdP;
    const int64_t st = bh * pn_count + p * A.dstate + n;  // [b, h, p, n]
    double hv = A.state_in ? (double)A.state_in[st] : 0.0;
    double* Sp = S + bh * nc * pn_count + np;
    const double* Ap = Ad + bh * nc;
    int c = 0;
    for (; c + 4 <= nc; c += 4) {  // four chunk loads in flight
        double sv[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) sv[k] = Sp[(int64_t)(c + k) * pn_count];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            Sp[(int64_t)(c + k) * pn_count] = hv;
            hv = __builtin_fma(Ap[c + k], hv, sv[k]);
        }
    }
    for (; c < nc; ++c) {
        const double sv = Sp[(int64_t)c * pn_count];
        Sp[(int64_t)c * pn_count] = hv;
        hv = __builtin_fma(Ap[c], hv, sv);
    }
    if (A.state_out)
        A.state_out[st] = (int32_t)__builtin_fmin(
            __builtin_fmax(__builtin_floor(hv + 0.5), -2147483648.0), 2147483647.0);
}

// ------------------------------------------------------------------ outputs
// Wave w owns the columns p = 16 w .. 16 w + 15 and every row t (4 tiles).
// G = C B^T on the int8 matrix cores; the decay mask L[t][s] = prod_{s<r<=t} a_r
// entry by entry as 2^(lg_t - lg_s) from prefix sums of log2 a, zero where a
// decay of 0 lies in (s, t] (counted by a second prefix sum: no division);
// M x (K = s <= t only) and C H_in^T (K = n, H_in^T streamed from the workspace)
// on the float64 matrix cores.
constexpr int kOutThreads = 256;

template <int N>
__global__ __launch_bounds__(kOutThreads) void ssd_chunk_out_kernel(ScanArgs A,
                                                                    const double* __restrict__ Hin,
                                                                    int nc) {
    constexpr int NR = N + 16;  // code row stride: 16-byte aligned rows, banks spread
    __shared__ double pre_s[Q], lg_s[Q], z_s[Q];
    __shared__ double M[Q][Q + 1];
    __shared__ __attribute__((aligned(16))) int8_t cs[Q][NR];
    __shared__ __attribute__((aligned(16))) int8_t xs[Q][kSsdP + 16];
    const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int H = (int)A.nheads;
    const int64_t L = A.len;
    const int t0 = c * Q;
    const int q = (int)(L - t0 < Q ? L - t0 : Q);
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, lr = lane & 15, lk = lane >> 4;
    // this wave's slice of H_in^T: [n][p = 16 wave + lr], one double per k-step
    constexpr int KS = N / 4, KH = KS / 2;  // k-steps over n, loaded in two halves
    const double* Hc = Hin + (((int64_t)b * H + h) * nc + c) * (int64_t)(kSsdP * N) +
                       lk * kSsdP + 16 * wave + lr;
    double hb[KH];
#pragma unroll
    for (int k = 0; k < KH; ++k) hb[k] = Hc[4 * k * kSsdP];
    // every lane: a and dt / 2^8 of token `lane` (padding 1, 0)
    double av = 1.0, dv = 0.0;
    if (lane < q) {
        const int64_t i = ((int64_t)b * L + t0 + lane) * H + h;
        av = (double)A.da_out[i] * 0x1p-16;
        dv = (double)A.dt_out[i] * 0x1p-8;
    }
    // B operands of G = C B^T straight from memory (the chunk's 8 KB sit in L2):
    // lane holds B codes [s = 16 j + lr][k0 + 8 lk .. + 7]; rows past the end are 0
    int64_t gb[4][N / 32];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int sr = 16 * j + lr;
        const int8_t* brow = A.bm + ((int64_t)b * L + t0 + sr) * N + 8 * lk;
#pragma unroll
        for (int k = 0; k < N / 32; ++k)
            gb[j][k] = sr < q ? *reinterpret_cast<const int64_t*>(brow + 32 * k) : (int64_t)0;
    }
    {  // staging: every global load of a thread issued before any LDS store
        constexpr int CL = Q * N / 16 / kOutThreads;  // 16-byte pieces of C
        int4 cv[CL];
#pragma unroll
        for (int k = 0; k < CL; ++k) {
            const int e = tid + kOutThreads * k, r = e / (N / 16), col = 16 * (e % (N / 16));
            const int64_t off = ((int64_t)b * L + t0 + r) * N + col;
            cv[k] = r < q ? *reinterpret_cast<const int4*>(A.cm + off) : int4{0, 0, 0, 0};
        }
        const int xr = tid >> 2, xc = 16 * (tid & 3);  // x: 64 rows of 64 bytes
        int4 xv = {0, 0, 0, 0};
        if (xr < q)
            xv = *reinterpret_cast<const int4*>(A.x + (((int64_t)b * L + t0 + xr) * H + h) * kSsdP + xc);
#pragma unroll
        for (int k = 0; k < CL; ++k) {
            const int e = tid + kOutThreads * k, r = e / (N / 16), col = 16 * (e % (N / 16));
            *reinterpret_cast<int4*>(&cs[r][col]) = cv[k];
        }
        *reinterpret_cast<int4*>(&xs[xr][xc]) = xv;
    }
    __syncthreads();
    {  // G = C B^T, exact: wave w takes the t tile w, every s
        i32x4 g[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) g[j] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < N / 32; ++k) {
            const int64_t ac = *reinterpret_cast<const int64_t*>(&cs[16 * wave + lr][32 * k + 8 * lk]);
#pragma unroll
            for (int j = 0; j < 4; ++j) g[j] = mfma_i8(ac, gb[j][k], g[j]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) M[16 * wave + 4 * lk + v][16 * j + lr] = (double)g[j][v];
    }
    if (wave == 0) {  // beside the other waves' products
        pre_s[lane] = wave_prefix_prod(av, lane);  // decay from the chunk start to t
        // prod_{s<r<=t} a_r = 2^(lg_t - lg_s) when no a_r in (s, t] is 0, i.e. z_t == z_s,
        // with lg, z the prefix sums of log2 a (a > 0) and of [a == 0]
        lg_s[lane] = wave_prefix_sum(av > 0.0 ? log2(av) : 0.0, lane);
        z_s[lane] = wave_prefix_sum(av > 0.0 ? 0.0 : 1.0, lane);
    }
    __syncthreads();
    // M[t][s] = G[t][s] prod_{s<r<=t} a_r dt_s for s <= t, 0 above: wave w takes the
    // rows t = w, w + 4, ..., lane s the column; every entry independent
    {
        const double lgs = lg_s[lane], zs = z_s[lane];
#pragma unroll 4
        for (int t = wave; t < Q; t += 4) {
            const bool live = lane <= t && z_s[t] == zs;
            const double mask = live ? exp2(lg_s[t] - lgs) : 0.0;
            M[t][lane] = M[t][lane] * mask * dv;
        }
    }
    __syncthreads();
    f64x4 yi[4], ye[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) yi[i] = ye[i] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int k = 0; k < KH; ++k) {  // C H_in^T, first half of n
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ye[i] = mfma_f64((double)cs[16 * i + lr][4 * k + lk], hb[k], ye[i]);
    }
#pragma unroll
    for (int k = 0; k < KH; ++k) hb[k] = Hc[4 * (KH + k) * kSsdP];  // second half in flight
    for (int s0 = 0; s0 < Q; s0 += 4) {  // M x: tile i only where s <= 16 i + 15
        const double bx = (double)xs[s0 + lk][16 * wave + lr];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (16 * i + 16 > s0) yi[i] = mfma_f64(M[16 * i + lr][s0 + lk], bx, yi[i]);
    }
#pragma unroll
    for (int k = 0; k < KH; ++k) {  // C H_in^T, second half of n
#pragma unroll
        for (int i = 0; i < 4; ++i)
            ye[i] = mfma_f64((double)cs[16 * i + lr][4 * (KH + k) + lk], hb[k], ye[i]);
    }
    const int ky = A.p[2] + A.p[3];
    const double sk = __builtin_ldexp(1.0, -ky);
    const double dq = (double)A.d_q16[h];
    const int p = 16 * wave + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int t = 16 * i + lk + 4 * v;
            if (t >= q) continue;
            const double acc = __builtin_fma(pre_s[t], ye[i][v], yi[i][v]);
            double y = __builtin_floor(__builtin_fma(acc, sk, 0.5));
            y = __builtin_fmin(__builtin_fmax(y, -0x1p62), 0x1p62);
            const double yd = __builtin_floor((dq * (double)xs[t][p] + 128.0) * 0x1p-8);
            A.y[(((int64_t)b * L + t0 + t) * H + h) * kSsdP + p] =
                (int32_t)__builtin_fmin(__builtin_fmax(y + yd, -2147483648.0), 2147483647.0);
        }
}

fm_status ssd_run(const ScanArgs& a, void* ws, hipStream_t s, hipEvent_t ev_start,
                  hipEvent_t ev_stop) {
    if (a.headdim != kSsdP)
        return fail(FM_ERR_SHAPE, "ssd scan: headdim %lld != %d", (long long)a.headdim, kSsdP);
    if (a.dstate != 64 && a.dstate != 128)
        return fail(FM_ERR_SHAPE, "ssd scan: dstate %lld not in {64, 128}", (long long)a.dstate);
    if (a.batch > 65535 || a.nheads > 65535)
        return fail(FM_ERR_SHAPE, "ssd scan: batch or nheads above 65535");
    fm_status st;
    if (!a.dt_ready && (st = scan_prep_run(a, s)) != FM_OK) return st;
    const int64_t nc64 = (a.len + Q - 1) / Q;
    if (nc64 > 0x7fffffff) return fail(FM_ERR_SHAPE, "ssd scan: too many chunks");
    const int nc = (int)nc64;
    const int64_t pn = a.headdim * a.dstate;
    double* S = (double*)ws;
    double* Ad = (double*)((char*)ws + align256((size_t)(a.batch * a.nheads * nc * pn) * sizeof(double)));
    const dim3 g(nc, (unsigned)a.nheads, (unsigned)a.batch);
    if (ev_start && hipEventRecord(ev_start, s) != hipSuccess)
        return fail(FM_ERR_HIP, "hipEventRecord(start) failed");
    if (a.dstate == 128) ssd_chunk_state_kernel<128><<<g, 256, 0, s>>>(a, S, Ad, nc);
    else ssd_chunk_state_kernel<64><<<g, 256, 0, s>>>(a, S, Ad, nc);
    if ((st = check_launch("ssd_chunk_state_kernel")) != FM_OK) return st;
    const int64_t elems = a.batch * a.nheads * pn;
    ssd_chunk_scan_kernel<<<(unsigned)((elems + 255) / 256), 256, 0, s>>>(a, S, Ad, nc, pn);
    if ((st = check_launch("ssd_chunk_scan_kernel")) != FM_OK) return st;
    if (a.dstate == 128) ssd_chunk_out_kernel<128><<<g, kOutThreads, 0, s>>>(a, S, nc);
    else ssd_chunk_out_kernel<64><<<g, kOutThreads, 0, s>>>(a, S, nc);
    if ((st = check_launch("ssd_chunk_out_kernel")) != FM_OK) return st;
    if (ev_stop && hipEventRecord(ev_stop, s) != hipSuccess)
        return fail(FM_ERR_HIP, "hipEventRecord(stop) failed");
    return FM_OK;
}

}  // namespace fm
