// Pipelined contraction: the same Y = A * B^T with fused bias epilogue as
// conv_gemm_kernel, but the A and B tiles are copied from global memory
// straight into LDS by buffer loads (buffer_load_dwordx4 ... lds), several
// tiles ahead of the MFMAs, in a ring of STAGES LDS stages.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract) names asynchronous data movement
// as one of its optimisations; on gfx950 the asynchronous path is the LDS-DMA
// form of the buffer load: a wave's 64 lanes each move 16 bytes into 1 KiB of
// LDS at M0 + 16*lane without passing through registers, and a lane whose
// offset lies outside the buffer writes zeros -- which is how the window
// loader produces the convolution's zero padding.
//
// The loads are issued from inline assembly so the compiler does not track
// them (its own tracking would wait for every outstanding LDS-DMA load before
// each LDS read); the kernel waits for them itself with s_waitcnt vmcnt and
// orders them with s_barrier:
//   iteration kt:  wait until tile kt has landed (the tiles after it may
//                  still be in flight) -> barrier (every wave's part of tile kt
//                  is visible, and every wave has finished reading the stage
//                  of tile kt-1) -> MFMAs on tile kt -> issue tile
//                  kt+STAGES-1 into the stage of tile kt-1
// or, with EARLY, the issue of tile kt+STAGES-1 right after the barrier and
// before the MFMAs on tile kt, which gives the loads STAGES-1 tiles' worth
// of MFMA time instead of STAGES-2 (the number of loads in flight at each
// wait is the same in both orders).
//
// LDS tiles use the same row swizzle as conv_gemm_kernel (swz_chunk).  Since a
// DMA writes LDS in lane order, the swizzle is applied on the global side:
// the lane that fills LDS chunk slot `slot` of row `row` loads global chunk
// swz_chunk(row, slot) (the XOR is its own inverse); for the tile shapes used
// that chunk is the same for all of a thread's loads.
#pragma once

#include "device_common.hpp"
#include "igemm.hpp"

namespace convlower {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource for raw (unformatted) 32-bit-offset access to [base, base+bytes).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4 r;
    r[0] = int32_t(uint32_t(a));
    r[1] = int32_t(uint32_t(a >> 32) & 0xffff);   // stride 0
    r[2] = int32_t(bytes);                          // num_records: offsets >= bytes read as 0
    r[3] = 0x00020000;                              // raw buffer, 32-bit data
    return r;
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

constexpr uint32_t kOutOfRange = 0x80000000u;   // any offset >= num_records (< 2^31) reads as zero

// floor(a / d) for 0 <= a < 2^22 and d >= 1, given rcp ~ 1/d (within a few
// ulp): float(a) is exact and a*rcp is within 1 of a/d, so one correction
// step on the remainder gives the quotient.  A few instructions instead of
// the ~30 of a general 32-bit division.
__device__ __forceinline__ int div_small(int a, int d, float rcp) {
    int q = int(float(a) * rcp);
    const int r = a - q * d;
    q += r >= d ? 1 : 0;
    q -= r < 0 ? 1 : 0;
    return q;
}

// The descriptor as the buffer-resource type of the LDS-DMA builtins.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t as_rsrc(i32x4 r) {
    const uint64_t a = (uint64_t(uint32_t(r[1]) & 0xffff) << 32) | uint32_t(r[0]);
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(a), 0, r[2], r[3]);
}

// 16 bytes from rsrc+voffset into LDS at m0 + 16*lane (m0 wave-uniform).
// Issued through the builtin, so that the compiler counts these loads in its
// own vmcnt bookkeeping: its waits for the registers of later ordinary loads
// then leave LDS-DMA loads issued after those registers' loads in flight.
// The compiler does not order LDS reads after these writes: every read of
// data they bring waits on vmcnt explicitly (wait_vmcnt) and, across
// waves, behind a barrier.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voffset, uint32_t m0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rsrc(rsrc), (__attribute__((address_space(3))) void*)uintptr_t(m0), 16,
                                             voffset, 0, 0, 0);
}

// Wait until at most N vector-memory loads of this wave are in flight (the
// s_waitcnt builtin, which the compiler's own vmcnt bookkeeping takes into
// account).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" : : : "memory"); }

// Swizzle mask of a thread's rows: for CPR chunks per row and NT threads,
// thread t fills rows j*(NT/CPR) + t/CPR, whose swizzle depends on t/CPR only
// (NT/CPR is a multiple of 8).
template <int CPR, int SWZ>
__device__ __forceinline__ int dma_chunk(int tid) {
    return swz_chunk<CPR, SWZ>(tid / CPR, tid % CPR);
}

// ---------------------------------------------------------------------------
// DMA sources.  init() fixes the thread's rows and its chunk, voff(j) is the
// byte offset of the thread's j-th 16-byte load of the current tile (or
// kOutOfRange), next() moves the contraction position by BK.

// Window of each output pixel gathered from NHWC x (C a multiple of VEC),
// contraction order (r, s, c).  Offsets are relative to the first image of
// the tile, so only that image range needs 32-bit offsets.
template <typename T, int ROWS, int BK, int NT, int SWZ = 0>
struct DmaWindowNHWC {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int CPR = BK / VEC;
    static constexpr int NL = ROWS * CPR / NT;      // loads per thread per tile
    static constexpr int RSTEP = NT / CPR;          // row distance between a thread's loads
    static_assert(ROWS * CPR % NT == 0, "whole wave loads");
    uint32_t nbase[NL];   // byte offset of the row's image
    int32_t h0[NL], w0[NL];
    bool ok[NL];
    int kk, c0, s, rr;
    i32x4 rsrc;

    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        int32_t n_first, p_, q_;
        decode_m(g, int32_t(row0 < g.M ? row0 : g.M - 1), n_first, p_, q_);
        const int64_t img = int64_t(g.H) * g.W * g.C;
        const T* base = static_cast<const T*>(g.a) + int64_t(n_first) * img;
        const int64_t n_imgs = g.M / g.PQ;
        rsrc = make_rsrc(base, uint32_t((n_imgs - n_first) * img * int64_t(sizeof(T)) < int64_t(0x7fffffff)
                                            ? (n_imgs - n_first) * img * int64_t(sizeof(T))
                                            : int64_t(0x7fffffff)));
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int64_t m = row0 + j * RSTEP + tid / CPR;
            ok[j] = m < g.M;
            int32_t n, p, q;
            decode_m(g, ok[j] ? int32_t(m) : 0, n, p, q);
            nbase[j] = uint32_t((n - n_first) * img * int64_t(sizeof(T)));
            h0[j] = p * g.sh - g.ph;
            w0[j] = q * g.sw - g.pw;
        }
        kk = dma_chunk<CPR, SWZ>(tid) * VEC;
        c0 = kk % g.C;
        const int rs = kk / g.C;
        s = rs % g.S;
        rr = rs / g.S;
    }
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j) const {
        const int h = h0[j] + rr * g.dh, w = w0[j] + s * g.dw;
        const bool in = ok[j] & (kk < g.Kc) & (unsigned(h) < unsigned(g.H)) & (unsigned(w) < unsigned(g.W));
        const uint32_t o = nbase[j] + uint32_t(((h * g.W + w) * g.C + c0) * int(sizeof(T)));
        return in ? o : kOutOfRange;
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        c0 += BK;
        while (c0 >= g.C) {
            c0 -= g.C;
            if (++s == g.S) {
                s = 0;
                ++rr;
            }
        }
    }
};

// As DmaWindowNHWC for C a multiple of BK: a tile then covers BK channels of
// one kernel tap (r, s) for every lane, so the tap and channel block are
// wave-uniform (scalar registers) and each load's offset is one add from a
// per-row base, two range checks and a select.
template <typename T, int ROWS, int BK, int NT, int SWZ = 0>
struct DmaWindowNHWCBlocked {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int CPR = BK / VEC;
    static constexpr int NL = ROWS * CPR / NT;
    static constexpr int RSTEP = NT / CPR;
    static_assert(ROWS * CPR % NT == 0, "whole wave loads");
    int32_t rowbase[NL];  // bytes: image base + (h0*W + w0)*C, plus this lane's channel chunk
    int32_t h0[NL], w0[NL];
    int cb, s, rr, kk;    // uniform: channel block start, tap, contraction position
    i32x4 rsrc;

    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        int32_t n_first, p_, q_;
        decode_m(g, int32_t(row0 < g.M ? row0 : g.M - 1), n_first, p_, q_);
        const int64_t img = int64_t(g.H) * g.W * g.C;
        const T* base = static_cast<const T*>(g.a) + int64_t(n_first) * img;
        const int64_t n_imgs = g.M / g.PQ;
        const int64_t bytes = (n_imgs - n_first) * img * int64_t(sizeof(T));
        rsrc = make_rsrc(base, uint32_t(bytes < int64_t(0x7fffffff) ? bytes : int64_t(0x7fffffff)));
        const int chunk = dma_chunk<CPR, SWZ>(tid);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int64_t m = row0 + j * RSTEP + tid / CPR;
            const bool ok = m < g.M;
            int32_t n, p, q;
            decode_m(g, ok ? int32_t(m) : 0, n, p, q);
            const int hv = p * g.sh - g.ph;
            w0[j] = q * g.sw - g.pw;
            rowbase[j] = int32_t((n - n_first) * img * int64_t(sizeof(T))) +
                         ((hv * g.W + w0[j]) * g.C + chunk * VEC) * int(sizeof(T));
            h0[j] = ok ? hv : -(1 << 28);   // rows past M never pass the range check
        }
        cb = 0;
        s = 0;
        rr = 0;
        kk = 0;
    }
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j) const {
        const int dh = rr * g.dh, dw = s * g.dw;
        const bool in = (unsigned(h0[j] + dh) < unsigned(g.H)) & (unsigned(w0[j] + dw) < unsigned(g.W)) & (kk < g.Kc);
        const int32_t o = rowbase[j] + ((dh * g.W + dw) * g.C + cb) * int(sizeof(T));
        return in ? uint32_t(o) : kOutOfRange;
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        cb += BK;
        if (cb == g.C) {
            cb = 0;
            if (++s == g.S) {
                s = 0;
                ++rr;
            }
        }
    }
};

// Rows of a strided matrix: lowered pixel rows (SEGMENTED for im2win strips)
// or filter rows.  Offsets are relative to the tile's first row.
template <typename T, int ROWS, int BK, bool PIXELS, bool SEGMENTED, int NT, int SWZ = 0>
struct DmaRows {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int CPR = BK / VEC;
    static constexpr int NL = (ROWS * CPR + NT - 1) / NT;
    static constexpr int RSTEP = NT / CPR;
    static_assert(ROWS * CPR % NT == 0 || ROWS * CPR < NT, "whole wave loads");
    uint32_t roff[NL];    // row start, bytes from the tile base
    bool ok[NL];
    int kk, t;
    uint32_t seg;         // bytes
    i32x4 rsrc;

    __device__ __forceinline__ int64_t row_offset(const GemmArgs& g, int64_t row) const {
        if (PIXELS) {
            int32_t n, p, q;
            decode_m(g, int32_t(row), n, p, q);
            return int64_t(n) * g.sN + int64_t(p) * g.sP + int64_t(q) * g.sQ;
        }
        return row * int64_t(g.ldb);
    }
    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        const int64_t nrows = PIXELS ? g.M : g.K;
        const int64_t first = row0 < nrows ? row0 : nrows - 1;
        const int64_t last = (row0 + ROWS - 1) < nrows ? row0 + ROWS - 1 : nrows - 1;
        const int64_t off0 = row_offset(g, first);
        // span of the tile: last row's start plus one full lowered row
        const int64_t span = (row_offset(g, last) - off0 + g.Kc +
                              (SEGMENTED ? int64_t(g.Kc / g.RCp) * (g.sS - g.RCp) : 0)) * int64_t(sizeof(T));
        const T* base = static_cast<const T*>(PIXELS ? g.a : g.b) + off0;
        rsrc = make_rsrc(base, uint32_t(span < int64_t(0x7fffffff) ? span : int64_t(0x7fffffff)));
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int64_t row = row0 + j * RSTEP + tid / CPR;
            ok[j] = (j * RSTEP + tid / CPR < ROWS) && row < nrows;
            roff[j] = uint32_t((row_offset(g, ok[j] ? row : first) - off0) * int64_t(sizeof(T)));
        }
        kk = dma_chunk<CPR, SWZ>(tid) * VEC;
        if (SEGMENTED) {
            t = kk % g.RCp;
            seg = uint32_t(int64_t(kk / g.RCp) * g.sS * int64_t(sizeof(T)));
        } else {
            t = kk;
            seg = 0;
        }
    }
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j) const {
        return (ok[j] && kk < g.Kc) ? roff[j] + seg + uint32_t(t * int(sizeof(T))) : kOutOfRange;
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        t += BK;
        if (SEGMENTED) {
            while (t >= g.RCp) {
                t -= g.RCp;
                seg += uint32_t(g.sS * int(sizeof(T)));
            }
        }
    }
};

// ---------------------------------------------------------------------------
// NT = 64*WGM*WGN threads (4 or 8 waves); two waves per SIMD either way
// (two 4-wave or one 8-wave workgroup per CU).
// EPI 0: bias add and store; 1: the ConvLSTM cell update (fp32 NCHW, BN = 64
// with WGN = 1).
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool NHWC_OUT, class ASrc, class BSrc,
          int EPI = 0, bool EARLY = false>
__global__ void __launch_bounds__(64 * WGM * WGN, 8 / (WGM * WGN)) conv_gemm_dma_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = WGM * WGN;
    constexpr int VEC = Vec<T>::n;
    constexpr int CPR = BK / VEC;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int KB = 4 * VEC;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;
    // DMA loads per thread per tile.  A narrow B tile (fewer than NT chunks)
    // is loaded by the first waves only, so the other waves issue fewer loads
    // and must wait with their own count.
    constexpr int B_WAVES = BN * CPR >= NT ? NW : (BN * CPR) / 64;
    constexpr int NLOADS = ASrc::NL + BSrc::NL;
    constexpr int NLOADS_NO_B = ASrc::NL;
    static_assert(BM * CPR % NT == 0, "A tile in whole workgroup loads");
    static_assert(BN * CPR >= NT || (BN * CPR) % 64 == 0, "B tile in whole wave loads");
    static_assert((NW == 4 || NW == 8) && BK % KB == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
    static_assert(STAGES >= 2, "at least double buffering");

    __shared__ __attribute__((aligned(16))) T smem[STAGES * STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const TileCoord tc = tile_coord(g, int((g.M + BM - 1) / BM));
    const int64_t m0 = int64_t(tc.m) * BM;
    const int n0 = tc.n * BN;

    ASrc la;
    BSrc lb;
    la.init(g, m0, tid);
    lb.init(g, n0, tid);

    // Split contraction (ksplit > 1): the workgroup of split z takes the
    // contraction tiles [z*per, min(nkt, (z+1)*per)); the loaders start there.
    // An empty range stores zeros.
    const int nkt_all = (g.Kc + BK - 1) / BK;
    int nkt = nkt_all;
    if (g.ksplit > 1) {
        const int per = (nkt_all + g.ksplit - 1) / g.ksplit;
        const int kt0 = tc.z * per;
        nkt = nkt_all - kt0 < per ? nkt_all - kt0 : per;
        for (int i = 0; i < kt0; ++i) {
            la.next(g);
            lb.next(g);
        }
    }

    const uint32_t lds0 = lds_offset(smem);
    // Issue one tile's loads into stage `st`: load j of wave w covers LDS chunk
    // slots [j*NT + w*64, +64) of the A (then B) region.
    auto issue = [&](int st) {
        const uint32_t a_base = lds0 + uint32_t(st * STAGE_ELEMS * sizeof(T));
        const uint32_t b_base = a_base + uint32_t(BM * BK * sizeof(T));
#pragma unroll
        for (int j = 0; j < ASrc::NL; ++j) dma16(la.rsrc, la.voff(g, j), a_base + uint32_t((j * NT + wave * 64) * 16));
#pragma unroll
        for (int j = 0; j < BSrc::NL; ++j) {
            if (wave < B_WAVES) dma16(lb.rsrc, lb.voff(g, j), b_base + uint32_t((j * NT + wave * 64) * 16));
        }
        la.next(g);
        lb.next(g);
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nkt) issue(st);

    const int frag_row = lane & 15;
    const int frag_chunk = lane >> 4;
    for (int kt = 0; kt < nkt; ++kt) {
        if (kt + STAGES - 2 < nkt) {
            // the STAGES-2 tiles after kt may stay in flight
            if (wave < B_WAVES)
                wait_vmcnt<(STAGES - 2) * NLOADS>();
            else
                wait_vmcnt<(STAGES - 2) * NLOADS_NO_B>();
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        // EARLY: the stage of tile kt-1 is free once every wave has passed this
        // barrier (each finished its MFMAs on tile kt-1, which waited for their
        // LDS reads), so the loads of tile kt+STAGES-1 can go out now.
        if constexpr (EARLY) {
            if (kt + STAGES - 1 < nkt) issue((kt + STAGES - 1) % STAGES);
        }
        const T* sA = smem + (kt % STAGES) * STAGE_ELEMS;
        const T* sB = sA + BM * BK;
        // All fragment reads of a step are issued ahead of its MFMAs
        // (sched_barrier), so the LDS latency is paid once per step.
#pragma unroll
        for (int kb = 0; kb < BK / KB; ++kb) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + frag_row;
                fa[i] = load16(sA + row * BK + swz_chunk<CPR>(row, kb * 4 + frag_chunk) * VEC);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 16 + frag_row;
                fb[j] = load16(sB + row * BK + swz_chunk<CPR>(row, kb * 4 + frag_chunk) * VEC);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = NHWC_OUT ? Mfma<T>::run(fb[j], fa[i], acc[i][j]) : Mfma<T>::run(fa[i], fb[j], acc[i][j]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // The next tile's loads go out after this tile's MFMAs are issued, so
        // their address arithmetic overlaps the MFMAs in flight.  Their stage
        // was last read in iteration kt-1, which every wave has left (barrier).
        if constexpr (!EARLY) {
            if (kt + STAGES - 1 < nkt) issue((kt + STAGES - 1) % STAGES);
        }
    }

    if constexpr (EPI == 1) {
        static_assert(sizeof(T) == 4 && !NHWC_OUT && BN == 64 && WGN == 1, "ConvLSTM epilogue tile");
        lstm_store_tile<WM, TM, TN>(g, acc, m0, n0, wm, lane);
    } else if (g.ksplit > 1) {
        // this split's fp32 partial sums, no bias, in the output layout
        GemmArgs h = g;
        h.y = static_cast<float*>(g.part) + int64_t(tc.z) * g.M * g.K;
        h.bias = nullptr;
        store_tile<float, BM, BN, WM, WN, TM, TN, NHWC_OUT>(h, acc, m0, n0, wm, wn, lane);
    } else {
        store_tile<T, BM, BN, WM, WN, TM, TN, NHWC_OUT>(g, acc, m0, n0, wm, wn, lane);
    }
}

// Sum of the split contraction's partials, in split order (deterministic),
// plus the bias, rounded to the storage type: y[i] = round(sum_z part[z][i] +
// bias[k(i)]), k(i) = i % K (NPQK) or (i / PQ) % K (NKPQ).  Four consecutive
// elements per thread.
struct SplitReduceArgs {
    const float* part;
    const void* bias;
    void* y;
    int64_t total;   // M*K
    int32_t K, PQ, ksplit, nhwc;
};

template <typename T>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(SplitReduceArgs a) {
    const T* __restrict__ bias = static_cast<const T*>(a.bias);
    T* __restrict__ y = static_cast<T*>(a.y);
    const bool vec = (a.total & 3) == 0;   // every split's slice 16-byte aligned
    for (int64_t i0 = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4; i0 < a.total;
         i0 += int64_t(gridDim.x) * 256 * 4) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (vec) {
            for (int z = 0; z < a.ksplit; ++z) {
                const f32x4 s = __builtin_bit_cast(f32x4, load16(a.part + z * a.total + i0));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += s[e];
            }
        } else {
            for (int z = 0; z < a.ksplit; ++z)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (i0 + e < a.total) v[e] += a.part[z * a.total + i0 + e];
        }
        T out[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t i = i0 + e;
            const int k = int(a.nhwc ? i % a.K : (i / a.PQ) % a.K);
            out[e] = from_f32<T>(v[e] + (bias ? to_f32(bias[k]) : 0.f));
        }
        if (vec) {
            if constexpr (sizeof(T) == 4) {
                store16(y + i0, u32x4{__float_as_uint(out[0]), __float_as_uint(out[1]), __float_as_uint(out[2]),
                                      __float_as_uint(out[3])});
            } else {
                union {
                    u32x2 u;
                    T e[4];
                } pk;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk.e[e] = out[e];
                *reinterpret_cast<u32x2*>(y + i0) = pk.u;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (i0 + e < a.total) y[i0 + e] = out[e];
        }
    }
}

}  // namespace convlower
