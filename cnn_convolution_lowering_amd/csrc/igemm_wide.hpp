// Wide-tile pipelined contraction for 16-bit storage: one wave per SIMD, each
// wave owning a large register tile (up to 128 x 128 outputs, 256 fp32
// accumulators) built from 32 x 32 x 16 MFMAs, with the LDS fragments of the
// next 16-deep contraction step read while the MFMAs of the current one run.
//
// Why a second pipelined kernel: with two waves per SIMD the register budget
// caps a wave's tile at 128 x 64, and the LDS then has to serve 12 KiB of
// fragment reads per 0.5 MFLOP of MFMA work, on top of the DMA writes of the
// tiles themselves.  A 128 x 128 wave tile reads 16 KiB per 1 MFLOP, so the
// LDS stays well below the MFMA time.  32 x 32 fragments halve the registers
// one step holds (four A and four B fragments per 16-deep step for a
// 128 x 128 wave tile), which leaves room to double-buffer them next to the
// accumulators.  With a single wave per SIMD nothing else hides the LDS
// latency, so the loop is software-pipelined instead:
//
//   step (kt, kb):  [at the last kb of a tile: wait until tile kt+1 has
//                   landed -> barrier -> issue the DMA of tile kt+STAGES-1
//                   into the stage of tile kt-1]
//                   -> read the fragments of the next step into the other
//                   register set -> MFMAs of this step.
//
// The stage overwritten by the DMA held tile kt-1, whose fragments every wave
// consumed (its MFMAs waited for them) before reaching this barrier.  Tiles
// and DMA sources are those of conv_gemm_dma_kernel, with the chunk swizzle
// for 32-row fragment reads (swz_chunk, SWZ = 1).  Source: "Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores" (abstract:
// asynchronous data movement on tensor-core convolution), restated for gfx950
// MFMA and LDS-DMA.
#pragma once

#include <type_traits>

#include "igemm_dma.hpp"

namespace convlower {

// Block index -> tile index such that the workgroups the dispatcher places on
// one XCD (round-robin, block b on XCD b % 8) own a contiguous range of
// tiles: neighbouring output rows share input rows, and each XCD has its own
// L2.  A bijection for any grid size.
__device__ __forceinline__ uint32_t xcd_tile(uint32_t bid, uint32_t nblk) {
    const uint32_t per = nblk / 8, rem = nblk % 8;
    const uint32_t xcd = bid % 8, idx = bid / 8;
    return xcd * per + (xcd < rem ? xcd : rem) + idx;
}

template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

template <typename T>
struct Mfma32;

template <>
struct Mfma32<_Float16> {
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

template <>
struct Mfma32<__bf16> {
    static __device__ __forceinline__ f32x16 run(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};

// Fused epilogue for 32 x 32 fragments fed (filter, pixel): acc[i][j][e] is
// output pixel m0 + wm*WM + i*32 + lane%32, channel
// n0 + wn*WN + j*32 + 8*(e/4) + 4*(lane/32) + e%4, so each group of four e is
// four consecutive channels of one NPQK row (one 8-byte store; 16 bytes for
// the fp32 partial sums of a split contraction).
template <typename T, int WM, int WN, int TM, int TN>
__device__ __forceinline__ void store_tile32_nhwc(const GemmArgs& g, const f32x16 (&acc)[TM][TN], int64_t m0, int n0,
                                                  int wm, int wn, int lane) {
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    const int kl = 4 * (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 32 + (lane & 31);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = n0 + wn * WN + j * 32 + 8 * q + kl;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e] + ((bias && k + e < g.K) ? to_f32(bias[k + e]) : 0.f);
                T* dst = y + m * g.K + k;
                if (k + 3 < g.K && (g.K & 3) == 0) {
                    if constexpr (sizeof(T) == 4) {   // fp32 partial sums of a split contraction
                        store16(dst, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                           __float_as_uint(v[3])});
                    } else {
                        union {
                            u32x2 u;
                            T e[4];
                        } pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(v[e]);
                        *reinterpret_cast<u32x2*>(dst) = pk.u;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (k + e < g.K) dst[e] = from_f32<T>(v[e]);
                }
            }
        }
    }
}

// ASrc / BSrc must be built with the SWZ = 1 swizzle (32-row fragment reads).
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, class ASrc, class BSrc>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) conv_gemm_wide_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = WGM * WGN;
    constexpr int VEC = Vec<T>::n;
    constexpr int CPR = BK / VEC;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int KB = 2 * VEC;          // contraction depth of one 32 x 32 x 16 step
    constexpr int KSUB = BK / KB;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;
    constexpr int B_WAVES = BN * CPR >= NT ? NW : (BN * CPR) / 64;
    constexpr int NLOADS = ASrc::NL + BSrc::NL;
    constexpr int NLOADS_NO_B = ASrc::NL;
    static_assert(sizeof(T) == 2, "16-bit storage");
    static_assert(BM * CPR % NT == 0, "A tile in whole workgroup loads");
    static_assert(BN * CPR >= NT || (BN * CPR) % 64 == 0, "B tile in whole wave loads");
    static_assert((NW == 2 || NW == 4 || NW == 8) && BK % KB == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(STAGES >= 3, "the DMA of a tile goes into the stage read two tiles earlier");
    static_assert((STAGES - 2) * NLOADS < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) T smem[STAGES * STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int tile_n = tile - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    ASrc la;
    BSrc lb;
    la.init(g, m0, tid);
    lb.init(g, n0, tid);
    // Split contraction (ksplit > 1): workgroup z = blockIdx.y takes the
    // contraction tiles [z*per, min(nkt, (z+1)*per)); the sources start
    // there.  An empty range stores zeros.
    const int nkt_all = (g.Kc + BK - 1) / BK;
    int nkt_split = nkt_all;
    if (g.ksplit > 1) {
        const int per = (nkt_all + g.ksplit - 1) / g.ksplit;
        const int kt0 = int(blockIdx.y) * per;
        nkt_split = nkt_all - kt0 < per ? nkt_all - kt0 : per;
        for (int i = 0; i < kt0; ++i) {
            la.next(g);
            lb.next(g);
        }
    }

    const uint32_t lds0 = lds_offset(smem);
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
    // Load `idx` of one tile's issue (A loads first, then B), into stage st;
    // the boundary step spreads these between its MFMAs.
    constexpr int NDMA = ASrc::NL + BSrc::NL;
    auto issue_one = [&](int st, auto idxc) __attribute__((always_inline)) {
        constexpr int idx = decltype(idxc)::value;
        const uint32_t a_base = lds0 + uint32_t(st * STAGE_ELEMS * sizeof(T));
        if constexpr (idx < ASrc::NL) {
            dma16(la.rsrc, la.voff(g, idx), a_base + uint32_t((idx * NT + wave * 64) * 16));
        } else {
            constexpr int j = idx - ASrc::NL;
            const uint32_t b_base = a_base + uint32_t(BM * BK * sizeof(T));
            if (wave < B_WAVES) dma16(lb.rsrc, lb.voff(g, j), b_base + uint32_t((j * NT + wave * 64) * 16));
        }
    };
    // Wait until at most N tiles of this wave's loads are still in flight.
    auto wait_tiles = [&](auto n) {
        constexpr int N = decltype(n)::value;
        if (wave < B_WAVES)
            wait_vmcnt<N * NLOADS>();
        else
            wait_vmcnt<N * NLOADS_NO_B>();
    };

    // Fragment read of sub-step kb from the stage at element offset `base`:
    // lane l takes row l%32 of each 32-row block and chunk 2*kb + l/32.
    const int frag_row = lane & 31;
    const int frag_chunk = lane >> 5;
    auto read = [&](u32x4 (&fa)[TM], u32x4 (&fb)[TN], int base, int kb) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = wm * WM + i * 32 + frag_row;
            fa[i] = load16(smem + base + row * BK + swz_chunk<CPR, 1>(row, kb * 2 + frag_chunk) * VEC);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WN + j * 32 + frag_row;
            fb[j] = load16(smem + base + BM * BK + row * BK + swz_chunk<CPR, 1>(row, kb * 2 + frag_chunk) * VEC);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    // (filter, pixel) operand order: the result rows are output channels.
    auto mfmas = [&](const u32x4 (&fa)[TM], const u32x4 (&fb)[TN]) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = Mfma32<T>::run(fb[j], fa[i], acc[i][j]);
    };

    const int nkt = nkt_split;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nkt) issue(st);
    // tile 0 landed (tiles 1 .. STAGES-2 may stay in flight)
    if (nkt >= STAGES - 1)
        wait_tiles(std::integral_constant<int, STAGES - 2>{});
    else
        wait_vmcnt<0>();
    lds_barrier();

    u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    read(fa0, fb0, 0, 0);

    // One contraction step: fragments of this step in (ca, cb); the next
    // step's go into (na, nb).  kb is the sub-step within tile kt, `stage`
    // the tile's stage index.
    int stage = 0;
    auto step = [&](int kt, auto kbc, const u32x4(&ca)[TM], const u32x4(&cb)[TN], u32x4(&na)[TM],
                    u32x4(&nb)[TN]) __attribute__((always_inline)) {
        constexpr int kb = decltype(kbc)::value;
        if constexpr (kb + 1 < KSUB) {
            read(na, nb, stage * STAGE_ELEMS, kb + 1);
        } else {
            // Tile kt+1 landed (the tiles after it may stay in flight).  The
            // barrier and the fragment reads run on the last tile too (they
            // then read a stale stage into registers nobody uses): with every
            // LDS read unconditional the compiler can count them exactly and
            // let the MFMAs below wait only for this step's fragments.
            if (kt + STAGES - 2 < nkt)
                wait_tiles(std::integral_constant<int, STAGES - 3>{});
            else
                wait_vmcnt<0>();
            lds_barrier();
            const int next = stage + 1 == STAGES ? 0 : stage + 1;
            read(na, nb, next * STAGE_ELEMS, 0);
            __builtin_amdgcn_sched_barrier(0);
            // The DMA of tile kt+STAGES-1 goes out one load after each MFMA:
            // with a single wave per SIMD, issuing them in one block would
            // leave the matrix core idle meanwhile.
            const bool more = kt + STAGES - 1 < nkt;
            const int st_dma = stage == 0 ? STAGES - 1 : stage - 1;
            static_for<TM * TN>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int i = idx / TN, j = idx % TN;
                acc[i][j] = Mfma32<T>::run(cb[j], ca[i], acc[i][j]);
                if constexpr (idx < NDMA) {
                    if (more) issue_one(st_dma, idxc);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            static_for<(NDMA > TM * TN ? NDMA - TM * TN : 0)>([&](auto rc) __attribute__((always_inline)) {
                if (more) issue_one(st_dma, std::integral_constant<int, TM * TN + decltype(rc)::value>{});
            });
            if (more) {
                la.next(g);
                lb.next(g);
            }
            __builtin_amdgcn_sched_barrier(0);
            stage = next;
            return;
        }
        __builtin_amdgcn_sched_barrier(0);
        mfmas(ca, cb);
        __builtin_amdgcn_sched_barrier(0);
    };
    // A tile's KSUB steps alternate the register sets.  With KSUB even every
    // tile starts from set 0.
    static_assert(KSUB % 2 == 0, "an even number of steps per tile");
    for (int kt = 0; kt < nkt; ++kt) {
        static_for<KSUB>([&](auto kbc) __attribute__((always_inline)) {
            constexpr int kb = decltype(kbc)::value;
            if constexpr ((kb & 1) == 0)
                step(kt, kbc, fa0, fb0, fa1, fb1);
            else
                step(kt, kbc, fa1, fb1, fa0, fb0);
        });
    }

    if (g.ksplit > 1) {
        // this split's fp32 partial sums, no bias
        GemmArgs h = g;
        h.y = static_cast<float*>(g.part) + int64_t(blockIdx.y) * g.M * g.K;
        h.bias = nullptr;
        store_tile32_nhwc<float, WM, WN, TM, TN>(h, acc, m0, n0, wm, wn, lane);
    } else {
        store_tile32_nhwc<T, WM, WN, TM, TN>(g, acc, m0, n0, wm, wn, lane);
    }
}

}  // namespace convlower
