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
#include <utility>

#include "fm_internal.hpp"

namespace fm {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;
constexpr int kGemmThreads = 256;
constexpr int kDepth = 3;          // k-steps whose global loads are in flight ahead of use

struct GemmParams {
    const int8_t* a;
    const int8_t* b;
    int64_t m, n, k;
    GemmEpilogue ep;
};

template <class F, int... Ss>
__device__ __forceinline__ void for_slots(std::integer_sequence<int, Ss...>, F&& f) {
    (f(std::integral_constant<int, Ss>{}), ...);
}

// The epilogue of a wave's TM x TN tiles of 16 x 16 (rows from row0, columns from
// col0; lane l holds rows 4*(l/16)+r, column l % 16 of each tile): int32 and / or
// dequantized float32 with the optional residual, and the column-range maximum
// (into a slot region under `slot_key`, or one word).
template <int TM, int TN>
__device__ __forceinline__ void tile_epilogue(const GemmParams& P, const v4i (&acc)[TM][TN],
                                              int64_t row0, int64_t col0, int lane,
                                              int64_t slot_key) {
    const GemmEpilogue& ep = P.ep;
    float sab = 0.0f;
    if (ep.out) sab = (*ep.s_a) * (*ep.s_b);
    float amax = 0.0f;
    // Whole tiles with float output only (almost every tile of a large product):
    // straight-line code, so the compiler counts the loads and stores in flight
    // exactly and never waits for a store's acknowledgement (on this chip stores
    // share the load counter); the residual, if any, never aliases the output.
    const bool whole = row0 + TM * 16 <= P.m && col0 + TN * 16 <= P.n && ep.out && !ep.acc;
    auto straight = [&](auto with_resid) {
        constexpr bool kRes = decltype(with_resid)::value;
        float* __restrict__ out = ep.out;
        const float* __restrict__ resid = ep.resid;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            float res[TN][4];
            if constexpr (kRes) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        res[j][r] = resid[(row0 + i * 16 + (lane >> 4) * 4 + r) * ep.ld_resid +
                                          col0 + j * 16 + (lane & 15)];
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int64_t col = col0 + j * 16 + (lane & 15);
                const bool in_max = col >= ep.amax_c0 && col < ep.amax_c1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t row = row0 + i * 16 + (lane >> 4) * 4 + r;
                    float o = (float)acc[i][j][r] * sab;
                    if constexpr (kRes) o = res[j][r] + o;
                    out[row * ep.ld_out + col] = o;
                    amax = in_max ? fmaxf(amax, fabsf(o)) : amax;
                }
            }
        }
    };
    if (whole && ep.resid) straight(std::true_type{});
    else if (whole) straight(std::false_type{});
    else
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        // the residual of this tile row, loaded as one batch before any store (the
        // output never aliases it; elements past the edge read a valid one, unused)
        float res[TN][4];
        if (ep.out && ep.resid) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                int64_t col = col0 + j * 16 + (lane & 15);
                col = col < P.n ? col : P.n - 1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int64_t row = row0 + i * 16 + (lane >> 4) * 4 + r;
                    row = row < P.m ? row : P.m - 1;
                    res[j][r] = ep.resid[row * ep.ld_resid + col];
                }
            }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int64_t col = col0 + j * 16 + (lane & 15);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = row0 + i * 16 + (lane >> 4) * 4 + r;
                if (row < P.m && col < P.n) {
                    int32_t v = acc[i][j][r];
                    if (ep.acc) ep.acc[row * ep.ld_acc + col] = v;
                    if (ep.out) {
                        float o = (float)v * sab;
                        if (ep.resid) o = res[j][r] + o;
                        ep.out[row * ep.ld_out + col] = o;
                        if (col >= ep.amax_c0 && col < ep.amax_c1) amax = fmaxf(amax, fabsf(o));
                    }
                }
            }
        }
    }
    if (ep.amax_slots) {
        amax = wave_max_f32(amax);
        if (lane == 0) slot_max(ep.amax_slots, slot_key, (int32_t)__float_as_uint(amax));
    } else if (ep.amax) {
        amax = wave_max_f32(amax);
        if (lane == 0 && amax > 0.0f) atomic_max_nonneg_f32(ep.amax, amax);
    }
}

// BM x BN x BK tiles (BK 64 or 128), 4 waves as 2 x 2, each (BM/2) x (BN/2) =
// TM x TN tiles of 16 x 16.  The global loads of k-steps kt+1 .. kt+kD are in
// flight (in a register ring) while step kt is multiplied from LDS; a 128-wide
// step runs two 64-wide rounds of products per barrier.
template <int BM, int BN, int BK>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(BK == 128 ? 2 : 3)))
void gemm_i8_kernel(GemmParams P) {
    constexpr int TM = BM / 32, TN = BN / 32;  // 16 x 16 tiles per wave
    constexpr int kRowsPerPass = kGemmThreads * 16 / BK;  // rows one load pass covers
    constexpr int RA = BM / kRowsPerPass, RB = BN / kRowsPerPass;
    constexpr int kD = BK == 128 ? 2 : kDepth;  // ring slots (the same bytes in flight)
    __shared__ __attribute__((aligned(16))) int8_t As[2][BM * BK];
    __shared__ __attribute__((aligned(16))) int8_t Bs[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    if (P.ep.pub_small && blockIdx.x == 0 && blockIdx.y == 0 && tid == 0)
        layer_publish(P.ep.pub_small, P.ep.pub_qp, P.ep.pub_cache_p);
    const int64_t m0 = (int64_t)blockIdx.y * BM;
    const int64_t n0 = (int64_t)blockIdx.x * BN;
    const int64_t K = P.k;

    // global -> register staging: each thread moves RA + RB pieces of 16 bytes
    const int ld_row = tid / (BK / 16);        // row inside a pass
    const int ld_col = (tid % (BK / 16)) * 16;  // byte offset inside the k slice
    const int8_t* pa[RA];
    const int8_t* pb[RB];
#pragma unroll
    for (int i = 0; i < RA; ++i) {
        int64_t r = m0 + ld_row + kRowsPerPass * i;
        r = r < P.m ? r : P.m - 1;  // rows past the edge: computed, never stored
        pa[i] = P.a + r * K + ld_col;
    }
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        int64_t r = n0 + ld_row + kRowsPerPass * i;
        r = r < P.n ? r : P.n - 1;
        pb[i] = P.b + r * K + ld_col;
    }
    v4i ring[kD][RA + RB];
    auto gload = [&](v4i* g, int64_t k0) {
#pragma unroll
        for (int i = 0; i < RA; ++i) g[i] = *reinterpret_cast<const v4i*>(pa[i] + k0);
#pragma unroll
        for (int i = 0; i < RB; ++i) g[RA + i] = *reinterpret_cast<const v4i*>(pb[i] + k0);
    };
    // BK-byte rows with their 16-byte granules XOR-swizzled by row (64-byte rows
    // by (r >> 2) & 3, 128-byte rows by (r >> 1) & 7): a store pass (16 lanes
    // over 4 or 2 rows) and a fragment read (16 rows, one granule) both touch 64
    // distinct banks
    auto swz = [](int row, int col) {
        const int g = BK == 64 ? ((row >> 2) & 3) : ((row >> 1) & 7);
        return row * BK + (col ^ (g << 4));
    };
    auto lstore = [&](const v4i* g, int buf) {
#pragma unroll
        for (int i = 0; i < RA; ++i)
            *reinterpret_cast<v4i*>(&As[buf][swz(ld_row + kRowsPerPass * i, ld_col)]) = g[i];
#pragma unroll
        for (int i = 0; i < RB; ++i)
            *reinterpret_cast<v4i*>(&Bs[buf][swz(ld_row + kRowsPerPass * i, ld_col)]) =
                g[RA + i];
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int64_t KT = K / BK;
    // Every load and LDS store of the pipeline is issued unconditionally (steps
    // past the end reload the last one), so the compiler counts the loads in
    // flight exactly and each step waits only for its own slot; only the
    // products are skipped past the end.
    auto kofs = [&](int64_t s) { return (s < KT ? s : KT - 1) * BK; };
    const bool live = P.m > 0 && P.n > 0;
    if (live) {
        gload(ring[0], 0);
        lstore(ring[0], 0);
        // steps 1 .. kD into slots 1 .. kD (mod kD)
        for_slots(std::make_integer_sequence<int, kD>{}, [&](auto S) {
            constexpr int s = decltype(S)::value + 1;
            gload(ring[s % kD], kofs(s));
        });
    }
    __syncthreads();
    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * 16;
    // step kt: multiply buffer kt & 1; store step kt + 1 (slot (kt+1) % kD)
    // into the other buffer; refill that slot with step kt + 1 + kD
    auto step = [&](int64_t kt, auto S) {
        constexpr int slot = (decltype(S)::value + 1) % kD;
        const int buf = (int)(kt & 1);
        if (kt < KT) {
#pragma unroll
            for (int kk = 0; kk < BK; kk += 64) {
                v4i af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = *reinterpret_cast<const v4i*>(
                        &As[buf][swz(wm * (BM / 2) + i * 16 + frag_row, kk + frag_k)]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf[j] = *reinterpret_cast<const v4i*>(
                        &Bs[buf][swz(wn * (BN / 2) + j * 16 + frag_row, kk + frag_k)]);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j],
                                                                          acc[i][j], 0, 0, 0);
            }
        }
        lstore(ring[slot], buf ^ 1);
        gload(ring[slot], kofs(kt + 1 + kD));
        __syncthreads();
    };
    for (int64_t kt = 0; kt < KT; kt += kD) {
        for_slots(std::make_integer_sequence<int, kD>{},
                  [&](auto S) { step(kt + decltype(S)::value, S); });
    }

    tile_epilogue<TM, TN>(P, acc, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane,
                          ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + wave);
}

// ---------------------------------------------------------------- large products
// M and N large (prefill over many tokens): 256 x 128 workgroup tiles, 4 waves
// as 2 x 2 of 128 x 64 (8 x 4 tiles of 16 x 16), 64-wide k-steps.  A and B move
// from global memory straight into LDS (16-byte direct loads: no registers, no
// LDS store instructions) through three stages, so the loads of steps kt+1 and
// kt+2 are in flight while step kt is multiplied; one barrier per step.  Each
// wave instruction fills 1 KB = 16 rows of 64 bytes, lane i taking row i / 4
// and the granule that the XOR swizzle puts at slot i % 4.  The swizzle
// (granule g of row r at slot g ^ h(r), h from bits 1-3 of r) keeps a fragment
// read free of bank conflicts whether the 16-byte reads of 8 or of 16 lanes are
// served together: rows r and r + 2 (8 lanes) and rows r and r + 4, r + 8,
// r + 12 (16 lanes) fall on different 16-byte bank groups.
// 72 KB of LDS and at most 128 accumulator registers per lane: two workgroups
// per CU, so one's epilogue stores overlap the other's products.
//
// Tile order: workgroup id i runs on XCD i % 8; tile q = (i % 8) * n8 + i / 8
// gives each XCD a contiguous range of q, and q runs through groups of 8 tile
// rows column by column, so the workgroups an XCD holds at once share the A
// rows and B columns they stream through its L2.
constexpr int kLdsStages = 3;

__device__ __forceinline__ int lds_swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }

// 16 bytes per lane from global memory straight into LDS: lane i's bytes land at
// dst + 16 i (dst wave-uniform)
__device__ __forceinline__ void lds_dma16(const int8_t* src, int8_t* dst) {
    __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}

template <int BM, int BN>
__global__ __launch_bounds__(kGemmThreads, 2) void gemm_i8_lds_kernel(GemmParams P) {
    constexpr int BK = 64;
    constexpr int TM = BM / 32, TN = BN / 32;
    static_assert(TM == 8 && TN == 4, "the fragment read block below is written for 8 x 4 tiles");
    constexpr int A_LD = BM * BK / 1024 / 4, B_LD = BN * BK / 1024 / 4;  // per wave and step
    constexpr int kA = BM * BK, kB = BN * BK;                             // bytes per stage
    __shared__ __attribute__((aligned(1024))) int8_t lds[kLdsStages * (kA + kB)];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t ntm = (P.m + BM - 1) / BM, ntn = (P.n + BN - 1) / BN;
    const int64_t ntiles = ntm * ntn, n8 = (ntiles + 7) / 8;
    const int64_t q = (int64_t)(blockIdx.x % 8) * n8 + blockIdx.x / 8;
    if (q >= ntiles) return;  // padding of the last XCD's range
    constexpr int64_t GM = 8;
    const int64_t grp = q / (GM * ntn), first = grp * GM;
    const int64_t rows_g = ntm - first < GM ? ntm - first : GM;
    const int64_t inner = q - grp * GM * ntn;
    const int64_t m0 = (first + inner % rows_g) * BM, n0 = (inner / rows_g) * BN;
    if (P.ep.pub_small && q == 0 && tid == 0)
        layer_publish(P.ep.pub_small, P.ep.pub_qp, P.ep.pub_cache_p);
    const int64_t K = P.k, KT = K / BK;

    // 64-byte rows, granule slot s of row r holds global granule s ^ lds_swz(r)
    const int ld_r = lane >> 2, ld_s = lane & 3;
    const int8_t* ga[A_LD];
    const int8_t* gb[B_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = (i * 4 + wave) * 16 + ld_r;  // row of the tile this lane fills
        int64_t gr = m0 + r;
        gr = gr < P.m ? gr : P.m - 1;  // rows past the edge: computed, never stored
        ga[i] = P.a + gr * K + ((ld_s ^ lds_swz(r)) << 4);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = (i * 4 + wave) * 16 + ld_r;
        int64_t gr = n0 + r;
        gr = gr < P.n ? gr : P.n - 1;
        gb[i] = P.b + gr * K + ((ld_s ^ lds_swz(r)) << 4);
    }
    // step s into stage st: A_LD + B_LD wave instructions of 1 KB
    auto issue = [&](int64_t s, int st) {
        const int64_t k0 = s * BK;
        int8_t* la = lds + st * (kA + kB);
        int8_t* lb = la + kA;
#pragma unroll
        for (int i = 0; i < A_LD; ++i) lds_dma16(ga[i] + k0, la + (i * 4 + wave) * 1024);
#pragma unroll
        for (int i = 0; i < B_LD; ++i) lds_dma16(gb[i] + k0, lb + (i * 4 + wave) * 1024);
    };
    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};
    // this lane's fragment row: tile i of A sits 1 KB after tile i - 1 (the swizzle
    // term depends on r % 16 only), likewise for B
    const int frag_row = lane & 15, frag_g = lane >> 4;
    const uint32_t lane_off = (uint32_t)(frag_row * BK + ((frag_g ^ lds_swz(frag_row)) << 4));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) int8_t*)lds;
    const uint32_t a_off = lds0 + (uint32_t)(wm * (BM / 2) * BK) + lane_off;
    const uint32_t b_off = lds0 + (uint32_t)kA + (uint32_t)(wn * (BN / 2) * BK) + lane_off;
    // The fragments of a step are read in one block that waits for them itself:
    // the compiler cannot tell these reads from the stages the direct loads are
    // still filling and would otherwise wait for every load in flight.
    auto compute = [&](int st) {
        const uint32_t sa = a_off + (uint32_t)(st * (kA + kB)), sb = b_off + (uint32_t)(st * (kA + kB));
        v4i a0, a1, a2, a3, a4, a5, a6, a7, b0, b1, b2, b3;
        asm volatile(
            "ds_read_b128 %0, %12\n\t"
            "ds_read_b128 %1, %12 offset:1024\n\t"
            "ds_read_b128 %2, %12 offset:2048\n\t"
            "ds_read_b128 %3, %12 offset:3072\n\t"
            "ds_read_b128 %4, %12 offset:4096\n\t"
            "ds_read_b128 %5, %12 offset:5120\n\t"
            "ds_read_b128 %6, %12 offset:6144\n\t"
            "ds_read_b128 %7, %12 offset:7168\n\t"
            "ds_read_b128 %8, %13\n\t"
            "ds_read_b128 %9, %13 offset:1024\n\t"
            "ds_read_b128 %10, %13 offset:2048\n\t"
            "ds_read_b128 %11, %13 offset:3072\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(a0), "=&v"(a1), "=&v"(a2), "=&v"(a3), "=&v"(a4), "=&v"(a5), "=&v"(a6),
              "=&v"(a7), "=&v"(b0), "=&v"(b1), "=&v"(b2), "=&v"(b3)
            : "v"(sa), "v"(sb)
            : "memory");
        const v4i af[TM] = {a0, a1, a2, a3, a4, a5, a6, a7};
        const v4i bf[TN] = {b0, b1, b2, b3};
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    };
    // vmcnt immediates: at most one step's loads (this wave's part) pending, or none
    constexpr int kPer = A_LD + B_LD;
    static_assert(kPer <= 15, "vmcnt immediate");
    constexpr int kWaitOne = kPer | (0x7 << 4) | (0xF << 8);
    constexpr int kWaitAll = 0 | (0x7 << 4) | (0xF << 8);
    issue(0, 0);
    if (KT > 1) issue(1, 1);
    for (int64_t kt = 0; kt < KT; kt += 3) {
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int64_t s = kt + u;
            if (s < KT) {
                // step s landed (this wave's part), then every wave's; stage (s+2)%3 was
                // last read at step s-1.  A plain barrier: the fence of __syncthreads
                // would also wait for the later steps' loads, which write LDS.
                if (s + 1 < KT) __builtin_amdgcn_s_waitcnt(kWaitOne);
                else __builtin_amdgcn_s_waitcnt(kWaitAll);
                asm volatile("s_barrier" ::: "memory");
                if (s + 2 < KT) issue(s + 2, (u + 2) % 3);
                compute(u);
            }
        }
    }
    tile_epilogue<TM, TN>(P, acc, m0 + wm * (BM / 2), n0 + wn * (BN / 2), lane, q * 4 + wave);
}

// ---------------------------------------------------------------- few rows (decode)
// M <= 64: weight traffic is the whole cost, so every workgroup streams its own
// 16*NT columns of B over the full K exactly once.  KW waves split K evenly;
// each keeps MT x NT (MT = ceil(M/16)) 16 x 16 accumulator tiles and issues up
// to kU 64-wide k-slices of loads at once.  The partial tiles are added through
// LDS (int32, exact in any order) and the epilogue is spread over all waves (each
// loads the residual of its share before the product).
constexpr int kSkU = 8;

// kMode 0: int8 A.  1: float A quantized on load; the columns hold z | xBC | dt
// of a one-token step: SiLU(z) in Q.16 goes to sz_out, xBC runs the conv step
// (power-of-two code, the 4-tap window from the conv cache shifted in place,
// SiLU, code of x / B / C, in the arithmetic of the conv kernel), dt is
// stored.  2: float A quantized on load, plain epilogue.
template <int MT, int NT, int KW, int kMode>
__global__ __launch_bounds__(64 * KW) void gemm_i8_few_rows_kernel(GemmParams P) {
    constexpr bool kAf = kMode != 0, kConv = kMode == 1;
    // float A: 4x the bytes per slice, held raw until the whole batch is issued
    constexpr int kU = kAf ? (MT == 1 ? 5 : (MT == 2 ? 2 : 1)) : kSkU;
    __shared__ __attribute__((aligned(16))) int32_t part[KW][MT][NT][64][4];
    __shared__ float wg_max[KW][2];      // per wave: max |out| (amax columns), max |xBC|
    __shared__ int32_t wg_pmax[KW][3];   // per wave: max |SiLU| of x, B, C
    __shared__ NauLds tab;
    if constexpr (kConv) nau_lds_init(tab);
    const GemmEpilogue& ep = P.ep;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t n0 = (int64_t)blockIdx.x * (16 * NT);
    const int di = (int)ep.d_inner, N = (int)ep.dstate, ch = di + 2 * N;

    // Epilogue units: (row tile t, column tile nt, row r of the lane's four),
    // one element per lane each; wave w takes units w, w + KW, ...
    constexpr int kUnits = MT * NT * 4, kUpw = (kUnits + KW - 1) / KW;
    // ---- the residual of this wave's units, loaded ahead of the product (rows
    // and columns past the edge read a valid element that is never used)
    float res[kUpw];
    if (!kConv && ep.resid) {
#pragma unroll
        for (int k = 0; k < kUpw; ++k) {
            const int un = wave + k * KW;
            const int t = un / (NT * 4), nt = (un / 4) % NT, r = un % 4;
            int64_t col = n0 + 16 * nt + (lane & 15);
            col = col < P.n ? col : P.n - 1;
            int64_t row = t * 16 + (lane >> 4) * 4 + r;
            row = row < P.m ? row : P.m - 1;
            res[k] = un < kUnits ? ep.resid[row * ep.ld_resid + col] : 0.0f;
        }
    }

    // ---- float A: the tensor scale from the row maxima (the same float ops everywhere)
    float c = 0.0f, s_a = 0.0f;
    if constexpr (kAf) {
        // m <= 64 row maxima: one per lane, one load round trip (max is exact)
        const float amax = wave_max_f32(lane < P.m ? ep.a_rowmax[lane] : 0.0f);
        if (ep.a_mode == FM_SCALE_DYNAMIC) c = amax == 0.0f ? 1.0f : 127.0f / amax;
        else c = ldexpf((float)ep.a_scoe, -ep.a_sshift);
        s_a = 1.0f / c;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            *ep.a_amax_out = amax;
            *ep.a_scale_out = s_a;
        }
    }
    if (ep.pub_small && blockIdx.x == 0 && threadIdx.x == 0)
        layer_publish(ep.pub_small, ep.pub_qp, ep.pub_cache_p);

    // ---- product
    // k range of this wave: slice ks = (wave + block) % KW, [ks*kq, ks*kq + kq): the
    // rotation spreads the workgroups' simultaneous reads of A over the slices
    const int64_t K = P.k, kq = K / KW;
    const int ks = (int)((wave + blockIdx.x) % KW);
    const int frag_row = lane & 15, frag_k = (lane >> 4) * 16;
    const int8_t* pb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        int64_t rb = n0 + 16 * nt + frag_row;
        rb = rb < P.n ? rb : P.n - 1;  // columns past the edge: computed, never stored
        pb[nt] = P.b + rb * K + ks * kq + frag_k;
    }
    int64_t aoff[MT];
    bool tap[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
        const int64_t ra0 = t * 16 + frag_row;
        tap[t] = kAf && ep.a_q_tap && blockIdx.x == 0 && ra0 < P.m;
        const int64_t ra = ra0 < P.m ? ra0 : P.m - 1;
        aoff[t] = ra * K + ks * kq + frag_k;
    }
    v4i acc[MT][NT];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[t][nt] = v4i{0, 0, 0, 0};
    // cnt <= kU slices: every load of the batch is issued before any use (the
    // optional code store may alias B, so no load may sit behind it)
    auto slices = [&](int64_t s0, int cnt) {
        v4i bf[kU][NT], af[kU][MT];
        float4 araw[kU][MT][4];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (u < cnt) {
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    bf[u][nt] = *reinterpret_cast<const v4i*>(pb[nt] + (s0 + u) * kBK);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    if constexpr (kAf) {
                        const float4* pa4 =
                            reinterpret_cast<const float4*>(ep.a_f + aoff[t] + (s0 + u) * kBK);
#pragma unroll
                        for (int e = 0; e < 4; ++e) araw[u][t][e] = pa4[e];
                    } else {
                        af[u][t] = *reinterpret_cast<const v4i*>(P.a + aoff[t] + (s0 + u) * kBK);
                    }
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of its uses
        if constexpr (kAf) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
                if (u < cnt)
#pragma unroll
                    for (int t = 0; t < MT; ++t) {
                        af[u][t] = v4i{(int)quant_pack4(araw[u][t][0], c),
                                       (int)quant_pack4(araw[u][t][1], c),
                                       (int)quant_pack4(araw[u][t][2], c),
                                       (int)quant_pack4(araw[u][t][3], c)};
                        if (tap[t])
                            *reinterpret_cast<v4i*>(ep.a_q_tap + aoff[t] + (s0 + u) * kBK) =
                                af[u][t];
                    }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u)
            if (u < cnt)
#pragma unroll
                for (int t = 0; t < MT; ++t)
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt)
                        acc[t][nt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[u][t], bf[u][nt],
                                                                           acc[t][nt], 0, 0, 0);
    };
    const int64_t steps = kq / kBK;
    int64_t s0 = 0;
    for (; s0 + kU <= steps; s0 += kU) slices(s0, kU);
    if (s0 < steps) slices(s0, (int)(steps - s0));
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            *reinterpret_cast<v4i*>(&part[wave][t][nt][lane][0]) = acc[t][nt];
    __syncthreads();

    // ---- epilogue: every wave, its units.  Phase 1 issues every load of the
    // wave's units (the conv window and weights with clamped, valid indices for
    // the units that do not use them); phase 2 computes and stores.
    float sab = 0.0f;
    if (ep.out) sab = (kAf ? s_a : *ep.s_a) * (*ep.s_b);
    int32_t uv[kUpw];
    int32_t xw[kUpw], xs0[kUpw], xs1[kUpw], xs2[kUpw], xpw[kUpw], xb[kUpw];
#pragma unroll
    for (int k = 0; k < kUpw; ++k) {
        const int un = wave + k * KW < kUnits ? wave + k * KW : kUnits - 1;
        const int t = un / (NT * 4), nt = (un / 4) % NT, r = un % 4;
        int32_t v = part[0][t][nt][lane][r];
#pragma unroll
        for (int w = 1; w < KW; ++w) v += part[w][t][nt][lane][r];
        uv[k] = v;
        if constexpr (kConv) {
            int64_t cx = n0 + 16 * nt + (lane & 15) - ep.amax_c0;
            cx = cx < 0 ? 0 : (cx >= ch ? ch - 1 : cx);
            int64_t row = t * 16 + (lane >> 4) * 4 + r;
            row = row < P.m ? row : P.m - 1;
            const int8_t* st = ep.conv_state + (row * ch + cx) * 3;
            xs0[k] = st[0];
            xs1[k] = st[1];
            xs2[k] = st[2];
            xw[k] = *reinterpret_cast<const int32_t*>(ep.conv_w_q + cx * 4);
            xpw[k] = ep.conv_p_w[cx];
            xb[k] = ep.conv_b_q16[cx];
        }
    }
    float amax = 0.0f, xmax = 0.0f;
    int32_t pmax[3] = {0, 0, 0};
#pragma unroll
    for (int k = 0; k < kUpw; ++k) {
        const int un = wave + k * KW;
        if (un >= kUnits) break;
        const int t = un / (NT * 4), nt = (un / 4) % NT, r = un % 4;
        const int64_t col0 = n0 + 16 * nt, col = col0 + (lane & 15);
        const int64_t row = t * 16 + (lane >> 4) * 4 + r;
        const int32_t v = uv[k];
        const bool ok = row < P.m && col < P.n;
        // column groups of 16 never straddle the z | xBC | dt boundaries
        if (kConv && col0 >= ep.amax_c0 && col0 < ep.amax_c1) {
            if (ok) {
                const int cx = (int)(col - ep.amax_c0);
                const int part_i = cx < di ? 0 : (cx < di + N ? 1 : 2);
                const int p_c = ep.conv_p[0];
                const int32_t w0 = (int8_t)(xw[k] & 0xFF), w1 = (int8_t)((xw[k] >> 8) & 0xFF),
                              w2 = (int8_t)((xw[k] >> 16) & 0xFF), w3 = (int8_t)(xw[k] >> 24);
                const double ascale = __builtin_ldexp(1.0, 16 - p_c - xpw[k]);
                const double oscale = __builtin_ldexp(1.0, ep.conv_p[1 + part_i] - 16);
                const int32_t xm3 = xs0[k], xm2 = xs1[k], xm1 = xs2[k];
                const float o = (float)v * sab;
                if (ep.write_xbc) ep.out[row * ep.ld_out + col] = o;
                xmax = fmaxf(xmax, fabsf(o));
                const int32_t xq = quant_xbc(o, ldexpf(1.0f, p_c));
                if (ep.xbc_q) ep.xbc_q[row * ch + cx] = (int8_t)xq;
                const int32_t acc4 = __mul24(w0, xm3) + __mul24(w1, xm2) + __mul24(w2, xm1) +
                                     __mul24(w3, xq);  // int8 products: 24-bit multiplies
                const double a = round_sat_d(__builtin_fma((double)acc4, ascale, (double)xb[k]));
                const int32_t sv = (int32_t)nau_silu_d(a, tab);
                const int32_t sa = sv < 0 ? -sv : sv;
                pmax[part_i] = sa > pmax[part_i] ? sa : pmax[part_i];
                // sat8(rshr(sv, 16 - p_part)): sv * 2^(p_part-16) is exact in float64
                const double q = __builtin_floor(__builtin_fma((double)sv, oscale, 0.5));
                int8_t* code = part_i == 0 ? ep.x_out + row * di + cx
                                           : (part_i == 1 ? ep.b_out + row * N + (cx - di)
                                                          : ep.c_out + row * N + (cx - di - N));
                *code = (int8_t)__builtin_fmin(__builtin_fmax(q, -127.0), 127.0);
                int8_t* st = ep.conv_state + (row * ch + cx) * 3;
                st[0] = (int8_t)xm2;
                st[1] = (int8_t)xm1;
                st[2] = (int8_t)xq;
            }
            continue;
        }
        if (kConv && col0 < ep.amax_c0) {  // z: SiLU(z) for the gate (Q.16 through the unit)
            if (ok) {
                const float o = (float)v * sab;
                if (ep.write_xbc) ep.out[row * ep.ld_out + col] = o;
                const double zq = f2d_sat(rintf(o * 65536.0f));
                ep.sz_out[row * di + col] = (float)nau_silu_d(zq, tab) * 0x1p-16f;
            }
            continue;
        }
        if (kConv && col0 >= ep.amax_c1) {  // dt: the raw value, dt and the decay
            if (ok) {
                const float o = (float)v * sab;
                ep.out[row * ep.ld_out + col] = o;
                const int64_t h = col - ep.amax_c1, nh = P.n - ep.amax_c1;
                const int32_t dt_in = f2i_sat(rintf((o + ep.dt_bias[h]) * 65536.0f));
                const int32_t dt = nau_softplus_f(dt_in, tab);
                ep.dt_out[row * nh + h] = dt;
                ep.da_out[row * nh + h] =
                    nau_exp_f(sat32(rshr((int64_t)dt * (int64_t)ep.a_q16[h], 16)), tab);
            }
            continue;
        }
        if (ok) {
            if (ep.acc) ep.acc[row * ep.ld_acc + col] = v;
            if (ep.out) {
                float o = (float)v * sab;
                if (ep.resid) o = res[k] + o;
                ep.out[row * ep.ld_out + col] = o;
                if (col >= ep.amax_c0 && col < ep.amax_c1) amax = fmaxf(amax, fabsf(o));
            }
        }
    }
    // the workgroup's maxima, then one atomic per quantity (into a slot region
    // where many workgroups would otherwise meet on one word)
    if (!kConv && !ep.amax && !ep.amax_slots) return;
    amax = wave_max_f32(amax);
    xmax = wave_max_f32(xmax);
#pragma unroll
    for (int i = 0; i < 3; ++i) pmax[i] = wave_max_i32(pmax[i]);
    if (lane == 0) {
        wg_max[wave][0] = amax;
        wg_max[wave][1] = xmax;
#pragma unroll
        for (int i = 0; i < 3; ++i) wg_pmax[wave][i] = pmax[i];
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < KW; ++w) {
            amax = fmaxf(amax, wg_max[w][0]);
            xmax = fmaxf(xmax, wg_max[w][1]);
            for (int i = 0; i < 3; ++i) pmax[i] = wg_pmax[w][i] > pmax[i] ? wg_pmax[w][i] : pmax[i];
        }
        if (kConv) {
            // slotted: hundreds of workgroups on one word each would serialize
            slot_max(ep.amax_slots, blockIdx.x, (int32_t)__float_as_uint(xmax));
            for (int i = 0; i < 3; ++i)
                slot_max(ep.conv_amax_slots + i * kSlotRegionWords, blockIdx.x, pmax[i]);
        } else if (ep.amax_slots) {
            slot_max(ep.amax_slots, blockIdx.x, (int32_t)__float_as_uint(amax));
        } else if (amax > 0.0f) {
            atomicMax(reinterpret_cast<unsigned int*>(ep.amax), __float_as_uint(amax));
        }
    }
}

template <int NT, int KW, int kMode>
static void launch_few_rows(const GemmParams& P, unsigned g, int mt, hipStream_t s) {
    switch (mt) {
        case 1: gemm_i8_few_rows_kernel<1, NT, KW, kMode><<<g, 64 * KW, 0, s>>>(P); break;
        case 2: gemm_i8_few_rows_kernel<2, NT, KW, kMode><<<g, 64 * KW, 0, s>>>(P); break;
        case 3: gemm_i8_few_rows_kernel<3, NT, KW, kMode><<<g, 64 * KW, 0, s>>>(P); break;
        default: gemm_i8_few_rows_kernel<4, NT, KW, kMode><<<g, 64 * KW, 0, s>>>(P); break;
    }
}

template <int kMode>
static void launch_few_rows_kw(const GemmParams& P, int64_t n, int mt, int kw, bool wide,
                               hipStream_t s) {
    const unsigned g1 = (unsigned)((n + 15) / 16), g4 = (unsigned)((n + 63) / 64);
    if (kw == 16) {  // mt == 1
        gemm_i8_few_rows_kernel<1, 1, 16, kMode><<<g1, 64 * 16, 0, s>>>(P);
    } else if (kw == 8) {
        if (wide) gemm_i8_few_rows_kernel<1, 4, 8, kMode><<<g4, 64 * 8, 0, s>>>(P);  // mt == 1
        else launch_few_rows<1, 8, kMode>(P, g1, mt, s);
    } else {
        launch_few_rows<1, 4, kMode>(P, g1, mt, s);
    }
}

// Codes of m <= 64 rotated rows with the tensor scale formed from their row
// maxima (the same float operations as the few-rows kernel's quantize-on-load:
// one pass here instead of one per workgroup of the product).  Thread = four
// consecutive elements.
__global__ __launch_bounds__(256) void quant_rows_kernel(const float* __restrict__ x,
                                                         const float* __restrict__ rowmax,
                                                         int64_t m, int64_t k, fm_scale_mode mode,
                                                         int32_t scoe, int32_t sshift,
                                                         uint32_t* __restrict__ q,
                                                         float* scale_out, float* amax_out) {
    const int lane = threadIdx.x & 63;
    const float amax = wave_max_f32(lane < m ? rowmax[lane] : 0.0f);
    float c;
    if (mode == FM_SCALE_DYNAMIC) c = amax == 0.0f ? 1.0f : 127.0f / amax;
    else c = ldexpf((float)scoe, -sshift);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *amax_out = amax;
        *scale_out = 1.0f / c;
    }
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < m * k / 4) q[i] = quant_pack4(reinterpret_cast<const float4*>(x)[i], c);
}

fm_status quant_rows_run(const float* x, const float* rowmax, int64_t m, int64_t k,
                         fm_scale_mode mode, int32_t scoe, int32_t sshift, int8_t* q,
                         float* scale_out, float* amax_out, hipStream_t s) {
    if (m < 1 || m > 64 || k % 4) return fail(FM_ERR_SHAPE, "quant_rows: m %lld k %lld",
                                              (long long)m, (long long)k);
    const int64_t n4 = m * k / 4;
    quant_rows_kernel<<<(unsigned)((n4 + 255) / 256), 256, 0, s>>>(
        x, rowmax, m, k, mode, scoe, sshift, reinterpret_cast<uint32_t*>(q), scale_out, amax_out);
    return check_launch("quant_rows_kernel");
}

fm_status gemm_run(const int8_t* a, const int8_t* b, int64_t m, int64_t n, int64_t k,
                   const GemmEpilogue& ep, hipStream_t s) {
    if (m == 0 || n == 0) return FM_OK;
    GemmParams P{a, b, m, n, k, ep};
    const bool conv = ep.conv_state != nullptr, af = ep.a_f != nullptr;
    if (conv && !af) return fail(FM_ERR_SHAPE, "gemm: the conv epilogue comes with float A");
    if (m <= 64 && k % (4 * kBK) == 0) {
        const int mt = (int)((m + 15) / 16);
        // as many k-splitting waves as keep at least 4 slices per wave (16 waves
        // only for one row tile: 1024 threads leave 128 registers per lane)
        int kw = 4;
        if (k % (16 * kBK) == 0 && k / (16 * kBK) >= 4 && mt == 1) kw = 16;
        else if (k % (8 * kBK) == 0 && k / (8 * kBK) >= 4) kw = 8;
        // float A is quantized again by every workgroup: with one row tile and
        // enough columns, 64 columns per workgroup cut that work by four
        const bool wide = af && mt == 1 && kw == 8 && (n + 63) / 64 >= 128;
        if (conv) launch_few_rows_kw<1>(P, n, mt, kw, wide, s);
        else if (af) launch_few_rows_kw<2>(P, n, mt, kw, wide, s);
        else launch_few_rows_kw<0>(P, n, mt, kw, false, s);
        return check_launch("gemm_i8_few_rows_kernel");
    }
    if (af) return fail(FM_ERR_SHAPE, "gemm: float A needs m <= 64, k %% 256 == 0");
    auto tiles = [&](int bm, int bn) { return ((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
    // large products: 256 x 128 tiles with direct-to-LDS loads, two per CU, as long
    // as every CU gets at least four of them
    const int64_t big = tiles(256, 128);
    if (big >= 4 * (int64_t)device_cus()) {
        const int64_t nwg = (big + 7) / 8 * 8;
        if (nwg >= ((int64_t)1 << 31)) return fail(FM_ERR_SHAPE, "gemm: %lld tiles", (long long)big);
        gemm_i8_lds_kernel<256, 128><<<(unsigned)nwg, kGemmThreads, 0, s>>>(P);
        return check_launch("gemm_i8_lds_kernel");
    }
    // the largest tiles that still give the chip's 256 CUs a workgroup each
    // 128-wide k-steps when k allows (half the barriers and waits per product)
    const bool k128 = k % 128 == 0;
    if (tiles(128, 128) >= 256) {
        dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 127) / 128));
        if (k128) gemm_i8_kernel<128, 128, 128><<<grid, kGemmThreads, 0, s>>>(P);
        else gemm_i8_kernel<128, 128, 64><<<grid, kGemmThreads, 0, s>>>(P);
    } else if (tiles(64, 128) >= 256) {
        dim3 grid((unsigned)((n + 127) / 128), (unsigned)((m + 63) / 64));
        if (k128) gemm_i8_kernel<64, 128, 128><<<grid, kGemmThreads, 0, s>>>(P);
        else gemm_i8_kernel<64, 128, 64><<<grid, kGemmThreads, 0, s>>>(P);
    } else {
        dim3 grid((unsigned)((n + 63) / 64), (unsigned)((m + 63) / 64));
        if (k128) gemm_i8_kernel<64, 64, 128><<<grid, kGemmThreads, 0, s>>>(P);
        else gemm_i8_kernel<64, 64, 64><<<grid, kGemmThreads, 0, s>>>(P);
    }
    return check_launch("gemm_i8_kernel");
}

}  // namespace fm
