// Strip-staged implicit contraction with the filter streamed into registers
// (16-bit NHWC, C a multiple of 32, at least two filter taps per row).
//
// The A side is the im2win strip of conv_strip_kernel: per filter row r and
// block of 32 channels, the input rows under the tile's output rows are
// copied once into LDS (LDS-DMA, zero padding from out-of-range offsets) and
// serve all S taps of that filter row ("Enabling Memory-efficient Im2win
// Convolution with Multi-precision Support on GPU CUDA and Tensor Cores",
// abstract).  The B side does not go through LDS at all: the filter is first
// packed (pack_filter_frag_kernel, lowering.hpp) into the order in which the MFMA consumes
// it, so each 32 x 16 filter fragment is one contiguous 1 KiB block and a
// wave loads it with a single 16-byte-per-lane buffer load.  That removes the
// filter tiles from the LDS traffic (which on gfx950 is the scarcer
// bandwidth) and, since nothing else in LDS changes from step to step, the
// per-step barrier: the workgroup synchronises only when it moves to the next
// strip.
//
// Per 32-deep step k (tap s, channel block cb, filter row r; s fastest), two
// 16-deep halves of TM*TN MFMAs each, with the memory operations of the
// next half spread one per MFMA:
//   half 0: A fragments of half 1 (LDS), filter fragments of step k+DB;
//   half 1: [last step of a strip: own strip loads landed, own LDS reads
//           done -> barrier] A fragments of step k+1, the rest of step
//           k+DB's filter fragments, and on the first step of a strip the
//           DMA of the strip after next into the buffer just released.
// Filter fragments live in a ring of DB+1 register sets, so the loop is
// unrolled DB+1 steps per trip to keep every index a compile-time constant.
#pragma once

#include "igemm_strip.hpp"

namespace convlower {

// 16 bytes per lane from a raw buffer into registers (a compiler-visible
// load: the compiler waits for it where the value is used).
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, int soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, int(voff), soff, 0));
}

// Waves whose accumulators take at most 128 registers (a 64 x 128 or
// smaller wave tile) fit two to a SIMD: the register budget asks for that,
// so one wave's waits and bookkeeping overlap the other's MFMAs.
template <int BM, int BN, int WGM, int WGN>
constexpr int strip_rb_min_blocks() {
    return (BM / WGM) * (BN / WGN) / 64 <= 128 ? 512 / (64 * WGM * WGN) : 1;
}

template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int DB>
__global__ void __launch_bounds__(64 * WGM * WGN, (strip_rb_min_blocks<BM, BN, WGM, WGN>()))
    conv_strip_rb_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int VEC = Vec<T>::n;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int STRIP_ELEMS = STRIP * VEC;
    constexpr int NR = DB + 1;   // filter register ring
    using ASrc = StripSrc<T, NT, STRIP>;
    constexpr int NLA = ASrc::NL;
    static_assert(sizeof(T) == 2 && VEC == 8, "16-bit storage");
    static_assert(STRIP % NT == 0 && WM % 32 == 0 && WN % 32 == 0 && DB >= 1, "tile shape");
    static_assert(NLA < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) T smem[2 * STRIP_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int tile_n = tile - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    const int32_t w_used = (g.Q - 1) * g.sw + (g.S - 1) * g.dw + 1;
    const int64_t m_last = (m0 + BM < g.M ? m0 + BM : g.M) - 1;
    const int32_t g0 = int32_t(m0 / g.Q);
    const int32_t t_rows = int32_t(m_last / g.Q) - g0 + 1;

    ASrc la;
    la.init(g, g0, t_rows, w_used, tid);

    int32_t srow[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 32 + (lane & 31);
        int32_t sr = 0;
        if (m < g.M) {
            const int32_t gr = int32_t(m / g.Q);
            sr = (gr - g0) * w_used + (int32_t(m) - gr * g.Q) * g.sw;
        }
        srow[i] = sr;
    }

    // Packed filter: fragment (nb, kk) at ((nb*KK + kk)*64 + lane)*16 bytes.
    const int KK = g.Kc / 16;
    const int NBt = (g.K + 31) / 32;
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.b), 0, int(int64_t(NBt) * KK * 1024), 0x00020000);
    const int nb0 = (n0 + wn * WN) / 32;
    // Per-lane offset of each fragment block (loop-invariant); the contraction
    // position goes into the scalar offset.  Blocks past the last output
    // channel re-read the last block: their results are never stored.
    uint32_t bfrag[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int nb = nb0 + j < NBt ? nb0 + j : NBt - 1;
        bfrag[j] = uint32_t((int64_t(nb) * KK * 64 + lane) * 16);
    }

    const uint32_t lds0 = lds_offset(smem);
    auto strip_load = [&](int buf, int j, int r, int cb) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, r, cb),
              lds0 + uint32_t(buf * STRIP_ELEMS * sizeof(T)) + uint32_t((j * NT + wave * 64) * 16));
    };
    const int frag_chunk = lane >> 5;
    // Element offset of the lane's A fragment of the first 16-deep half of a
    // step (strip buffer buf, tap s).  The second half's fragment is the
    // next chunk pair of the same row: its swizzled chunk index differs in
    // bit 1 only (the XOR mask touches bits 0-1 of the chunk, and the first
    // half's chunk is 0 or 1), i.e. its offset is this one XOR 2*VEC (buffer
    // starts are multiples of 2048 elements, rows of 4*VEC).  So each step
    // computes one offset per fragment and the second half reuses it.
    static_assert(STRIP_ELEMS % 2048 == 0, "offset bit 4 belongs to the chunk");
    auto a_off = [&](int i, int buf, int s) __attribute__((always_inline)) {
        const int row = srow[i] + s * g.dw;
        return buf * STRIP_ELEMS + (row * 4 + swz_chunk<4, 1>(row, frag_chunk)) * VEC;
    };
    int aoff[TM];   // first-half offsets of the current step
    // Filter fragments of step position `kpos16` (contraction index / 16) for both halves.
    auto load_b = [&](u32x4 (&fb)[2][TN], int kpos16) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[h][j] = buffer_load16(brsrc, bfrag[j], (kpos16 + h) * 1024);
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int S = g.S, CB = g.C / 32;
    const int nsteps = g.R * CB * S;
    const int nstrips = g.R * CB;

    // Prologue: strip 0 (and strip 1) into LDS, filter fragments of steps 0 .. DB-1.
#pragma unroll
    for (int j = 0; j < NLA; ++j) strip_load(0, j, 0, 0);
    int sr1 = 0, scb1 = 1;     // (r, cb) of strip 1
    if (scb1 == CB) {
        scb1 = 0;
        ++sr1;
    }
    if (nstrips > 1) {
#pragma unroll
        for (int j = 0; j < NLA; ++j) strip_load(1, j, sr1, scb1);
    }
    u32x4 fb[NR][2][TN];
    StepPos pb{0, 0, 0};       // position of the next filter fragments to load
    static_for<DB>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        const bool more = d < nsteps;
        load_b(fb[d], more ? ((pb.r * S + pb.s) * g.C + pb.cb * 32) / 16 : 0);
        if (more) pb.advance(S, CB);
    });
    // everything in flight landed (once per kernel: strips 0 and 1, filter steps 0 .. DB-1)
    wait_vmcnt<0>();
    lds_barrier();

    u32x4 fa0[TM], fa1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        aoff[i] = a_off(i, 0, 0);
        fa0[i] = load16(smem + aoff[i]);
    }

    StepPos pc{0, 0, 0};      // step k
    int strip_k = 0;
    int next_strip = 2;       // next strip to load
    int nsr = sr1, ncb = scb1 + 1;
    if (ncb == CB) {
        ncb = 0;
        ++nsr;
    }

    // One step with the filter fragments of this step in register set RC and
    // the set that receives step k+DB's fragments, RL.
    // One step: every memory operation sits between two MFMAs (one per
    // MFMA), so its issue and address arithmetic overlap the matrix core
    // instead of stalling it -- with one wave per SIMD nothing else would.
    //   half 0 (MFMAs on fa0, fb[RC][0]): A fragments of half 1 -> fa1,
    //     then the first half of step k+DB's filter fragments -> fb[RL][0];
    //   half 1 (MFMAs on fa1, fb[RC][1]): [strip boundary: wait, barrier]
    //     A fragments of step k+1 -> fa0, the rest of step k+DB's filter
    //     fragments -> fb[RL][1], then the strip loads (first step of a strip).
    auto step = [&](int k, auto rcc) __attribute__((always_inline)) {
        constexpr int RC = decltype(rcc)::value;
        constexpr int RL = (RC + DB) % NR;
        constexpr int NM = TM * TN;
        const bool more = k + DB < nsteps;
        // Past the end the loads repeat position 0 into a set nobody reads:
        // unconditional loads keep the compiler's count of them exact.
        const int kpos_b = more ? ((pb.r * S + pb.s) * g.C + pb.cb * 32) / 16 : 0;
        // ---- half 0
        static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
            constexpr int idx = decltype(idxc)::value;
            constexpr int i = idx / TN, j = idx % TN;
            acc[i][j] = Mfma32<T>::run(fb[RC][0][j], fa0[i], acc[i][j]);
            if constexpr (idx < TM) {
                fa1[idx] = load16(smem + (aoff[idx] ^ (2 * VEC)));
            } else if constexpr (idx < TM + TN) {
                fb[RL][0][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kpos_b * 1024);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(TM + TN > NM ? TM + TN - NM : 0)>([&](auto rc) __attribute__((always_inline)) {
            constexpr int idx = NM + decltype(rc)::value;
            if constexpr (idx < TM)
                fa1[idx] = load16(smem + (aoff[idx] ^ (2 * VEC)));
            else
                fb[RL][0][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kpos_b * 1024);
        });
        __builtin_amdgcn_sched_barrier(0);
        // ---- half 1
        StepPos pn = pc;
        pn.advance(S, CB);
        const bool last = k + 1 == nsteps;
        const bool new_strip = !last && pn.s == 0;
        if (new_strip) {
            // Strip strip_k+1 (in the other buffer) must have landed for every
            // wave, and every wave must be done reading this strip's buffer
            // before it is refilled.  Its loads went out at the end of the
            // previous strip boundary; the wave's loads since then are filter
            // fragments only: 2*TN per step of this strip, less the TN of this
            // half not yet issued, (2S-1)*TN in all.  Loads complete in order,
            // so waiting until at most that many are in flight waits for the
            // strip and nothing later; the wait keeps as many of the filter
            // loads in flight as its 6-bit count allows, so the filter
            // prefetch does not drain at every strip.
            if (S >= 8)
                wait_vmcnt<(15 * TN < 63 ? 15 * TN : 63)>();
            else if (S >= 4)
                wait_vmcnt<7 * TN>();
            else
                wait_vmcnt<2 * TN>();
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
            lds_barrier();
        }
        const int strip_n = new_strip ? strip_k + 1 : strip_k;
        const int buf_n = (last ? strip_k : strip_n) & 1, s_n = last ? pc.s : pn.s;
        const bool do_strip = new_strip && next_strip < nstrips;
        __builtin_amdgcn_sched_barrier(0);
        static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
            constexpr int idx = decltype(idxc)::value;
            constexpr int i = idx / TN, j = idx % TN;
            acc[i][j] = Mfma32<T>::run(fb[RC][1][j], fa1[i], acc[i][j]);
            if constexpr (idx < TM) {
                aoff[idx] = a_off(idx, buf_n, s_n);
                fa0[idx] = load16(smem + aoff[idx]);
            } else if constexpr (idx < TM + TN) {
                fb[RL][1][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], (kpos_b + 1) * 1024);
            } else if constexpr (idx - TM - TN < NLA) {
                if (do_strip) strip_load(next_strip & 1, idx - TM - TN, nsr, ncb);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(TM + TN + NLA > NM ? TM + TN + NLA - NM : 0)>([&](auto rc) __attribute__((always_inline)) {
            constexpr int idx = NM + decltype(rc)::value;
            if constexpr (idx < TM) {
                aoff[idx] = a_off(idx, buf_n, s_n);
                fa0[idx] = load16(smem + aoff[idx]);
            } else if constexpr (idx < TM + TN)
                fb[RL][1][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], (kpos_b + 1) * 1024);
            else if (do_strip)
                strip_load(next_strip & 1, idx - TM - TN, nsr, ncb);
        });
        __builtin_amdgcn_sched_barrier(0);
        if (more) pb.advance(S, CB);
        if (do_strip) {
            ++next_strip;
            if (++ncb == CB) {
                ncb = 0;
                ++nsr;
            }
        }
        pc = pn;
        strip_k = strip_n;
    };

    // Whole trips first: no step of a trip is conditional, so the compiler's
    // count of the filter loads in flight is the same at every trip start and
    // its waits stay exact; then the remaining steps.
    int k = 0;
    for (; k + NR <= nsteps; k += NR) {
        static_for<NR>([&](auto rcc) __attribute__((always_inline)) { step(k + decltype(rcc)::value, rcc); });
    }
    static_for<NR - 1>([&](auto rcc) __attribute__((always_inline)) {
        constexpr int RC = decltype(rcc)::value;
        if (k + RC < nsteps) step(k + RC, rcc);
    });

    // Fused epilogue: bias for this lane's channels loaded in one batch.
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    const int kl = 4 * (lane >> 5);
    float bv[TN][4][4];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int k = n0 + wn * WN + j * 32 + 8 * q + kl;
            if (bias && (g.K & 3) == 0 && k + 3 < g.K) {
                // four consecutive channels, 8-byte aligned (k and K multiples of 4)
                union {
                    u32x2 u;
                    T e[4];
                } pk;
                pk.u = *reinterpret_cast<const u32x2*>(bias + k);
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[j][q][e] = to_f32(pk.e[e]);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[j][q][e] = (bias && k + e < g.K) ? to_f32(bias[k + e]) : 0.f;
            }
        }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 32 + (lane & 31);
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = n0 + wn * WN + j * 32 + 8 * q + kl;
                T* dst = y + m * g.K + k;
                if (k + 3 < g.K && (g.K & 3) == 0) {
                    union {
                        u32x2 u;
                        T e[4];
                    } pk;
#pragma unroll
                    for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(acc[i][j][4 * q + e] + bv[j][q][e]);
                    *reinterpret_cast<u32x2*>(dst) = pk.u;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (k + e < g.K) dst[e] = from_f32<T>(acc[i][j][4 * q + e] + bv[j][q][e]);
                }
            }
        }
    }
}

}  // namespace convlower
