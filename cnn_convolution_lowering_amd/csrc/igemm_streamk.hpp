// Stream-K form of the pipelined contraction, for layers whose output tiles
// cannot fill the GPU evenly (a few hundred 128 x 128 tiles on 256 CUs).
//
// The work is the (tile, contraction step) pairs in tile-major order; a
// persistent grid of G workgroups (two per CU) takes equal contiguous ranges
// of it, so every CU does the same share however many tiles there are
// ("GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
// Extension", section "Engineering Challenges": tile sizes change occupancy
// and work distribution).  A range covers whole tiles in the middle and a
// piece of a tile at either end.  For a tile split between workgroups:
//   - the workgroups whose ranges start inside it (a later piece of its
//     contraction) compute that piece first thing, store the fp32 sums in
//     their own slot of the workspace and publish them with a flag that
//     carries this launch's epoch;
//   - the workgroup whose range ends inside it (the first piece, from
//     contraction step 0) computes that piece last, then adds the later
//     pieces' sums in contraction order and stores the tile with the bias.
// The sum order is fixed by the static partition, so results do not depend
// on timing.  The owner's wait targets pieces computed at the start of
// other workgroups' runs, which the grid (no larger than the GPU holds at
// once) has started with it; the wait is still bounded: a tile whose pieces
// do not arrive in about a second is written as NaN, never a hang.
//
// Each piece is one pass of the early-issue LDS-DMA pipeline of
// conv_gemm_dma_kernel over its contraction steps.  A slot stores the
// workgroup's accumulators in register order (lane-major per fragment), and
// the owner reads them back in the same order, so no layout change is needed.
// (A first form published the slots with release / acquire fences at device
// scope: on this multi-XCD GPU those write back and invalidate a whole XCD's
// L2 and made the layer six times slower.)
#pragma once

#include "igemm_dma.hpp"

namespace convlower {

struct StreamKArgs {
    float* part;          // grid slots of BM*BN fp32 sums
    uint32_t* flags;      // grid flags, flag[v] == epoch: slot v holds this launch's sums
    uint32_t epoch;       // nonzero, different for every launch
    int32_t tiles;        // output tiles (tiles_n per tile row)
    int32_t nkt;          // contraction steps per tile
    int32_t grid;         // workgroups
};

constexpr uint32_t kStreamKSpinLimit = 1u << 24;   // s_sleep 2 (~128 cycles) each: about a second
constexpr int kDeviceScope = 16;                     // buffer cache policy: sc1 (device scope)

// At least two workgroups per CU (16 waves of 8 -- at most 128 VGPRs -- or
// 16 of 4): the grid of two per CU is then resident at once.
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool NHWC_OUT, class ASrc, class BSrc>
__global__ void __launch_bounds__(64 * WGM * WGN, 16 / (WGM * WGN))
    conv_gemm_streamk_kernel(GemmArgs g, StreamKArgs sk) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = WGM * WGN;
    constexpr int VEC = Vec<T>::n;
    constexpr int CPR = BK / VEC;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int KB = 4 * VEC;
    constexpr int STAGE_ELEMS = (BM + BN) * BK;
    constexpr int B_WAVES = BN * CPR >= NT ? NW : (BN * CPR) / 64;
    constexpr int NLOADS = ASrc::NL + BSrc::NL;
    constexpr int NLOADS_NO_B = ASrc::NL;
    static_assert(BM * CPR % NT == 0, "A tile in whole workgroup loads");
    static_assert(BN * CPR >= NT || (BN * CPR) % 64 == 0, "B tile in whole wave loads");
    static_assert((NW == 4 || NW == 8) && BK % KB == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
    static_assert(STAGES >= 2, "at least double buffering");

    __shared__ __attribute__((aligned(16))) T smem[STAGES * STAGE_ELEMS];
    __shared__ int s_fail;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int frag_row = lane & 15;
    const int frag_chunk = lane >> 4;
    const uint32_t lds0 = lds_offset(smem);

    // The workgroup's rank in the work: workgroups are dealt to the eight
    // XCDs round robin, so ranks go to XCDs in contiguous blocks -- the pieces
    // of a split tile, and neighbouring tiles, then mostly run on one XCD and
    // share its L2.
    int v;
    {
        const int x = int(blockIdx.x) % kXcds, i = int(blockIdx.x) / kXcds;
        const int q = sk.grid / kXcds, r = sk.grid - q * kXcds;
        v = x * q + (x < r ? x : r) + i;
    }
    const int64_t total = int64_t(sk.tiles) * sk.nkt;
    auto start_of = [&](int w) { return int64_t(w) * total / sk.grid; };   // first unit of workgroup w
    const int64_t u_end = start_of(v + 1);

    ASrc la;
    BSrc lb;
    f32x4 acc[TM][TN];
    // The sum slots, read and written only with device-scope accesses
    // (cache policy sc1): coherent across XCDs without flushing or
    // invalidating any cache, which would throw away the operand tiles other
    // workgroups have in their XCD's L2.  Together with the flags (relaxed
    // device-scope atomics) and the wait for the slot stores to complete before
    // the flag is set, this orders a slot's data before its flag.
    const __amdgpu_buffer_rsrc_t prsrc =
        __builtin_amdgcn_make_buffer_rsrc(sk.part, 0, int(sk.grid * (BM * BN * 4)), 0x00020000);

    auto issue = [&](int st) __attribute__((always_inline)) {
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

    for (int64_t u = start_of(v); u < u_end;) {
        const int t = int(u / sk.nkt);
        const int kb = int(u - int64_t(t) * sk.nkt);
        const int64_t tile_end = int64_t(t + 1) * sk.nkt;
        const int ke = int((u_end < tile_end ? u_end : tile_end) - int64_t(t) * sk.nkt);
        u = int64_t(t) * sk.nkt + ke;
        const int tile_m = t / g.tiles_n;
        const int tile_n = t - tile_m * g.tiles_n;
        const int64_t m0 = int64_t(tile_m) * BM;
        const int n0 = tile_n * BN;
        const int nkt = ke - kb;

        // The previous piece's last LDS reads are done everywhere before its
        // stages are refilled.
        asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
        lds_barrier();
        la.init(g, m0, tid);
        lb.init(g, n0, tid);
        for (int i = 0; i < kb; ++i) {
            la.next(g);
            lb.next(g);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
        for (int st = 0; st < STAGES - 1; ++st)
            if (st < nkt) issue(st);
        for (int kt = 0; kt < nkt; ++kt) {
            if (kt + STAGES - 2 < nkt) {
                if (wave < B_WAVES)
                    wait_vmcnt<(STAGES - 2) * NLOADS>();
                else
                    wait_vmcnt<(STAGES - 2) * NLOADS_NO_B>();
            } else {
                wait_vmcnt<0>();
            }
            lds_barrier();
            if (kt + STAGES - 1 < nkt) issue((kt + STAGES - 1) % STAGES);
            const T* sA = smem + (kt % STAGES) * STAGE_ELEMS;
            const T* sB = sA + BM * BK;
#pragma unroll
            for (int kbb = 0; kbb < BK / KB; ++kbb) {
                u32x4 fa[TM], fb[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    const int row = wm * WM + i * 16 + frag_row;
                    fa[i] = load16(sA + row * BK + swz_chunk<CPR>(row, kbb * 4 + frag_chunk) * VEC);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    const int row = wn * WN + j * 16 + frag_row;
                    fb[j] = load16(sB + row * BK + swz_chunk<CPR>(row, kbb * 4 + frag_chunk) * VEC);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = NHWC_OUT ? Mfma<T>::run(fb[j], fa[i], acc[i][j])
                                             : Mfma<T>::run(fa[i], fb[j], acc[i][j]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        if (kb > 0) {
            // A later piece of tile t: sums to this workgroup's slot (device-scope
            // stores, written through to where every XCD sees them), completed by
            // every thread, then the flag.
            const uint32_t sbase = uint32_t(v) * uint32_t(BM * BN * 4);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), prsrc,
                                                           int(sbase + uint32_t(((i * TN + j) * NT + tid) * 16)), 0,
                                                           kDeviceScope);
            asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_store(sk.flags + v, sk.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            continue;
        }
        if (ke < sk.nkt) {
            // The first piece of tile t: add the later pieces, in contraction order.
            for (int w = v + 1; w < sk.grid && start_of(w) < tile_end; ++w) {
                if (tid == 0) {
                    int fail = 0;
                    uint32_t spins = 0;
                    while (__hip_atomic_load(sk.flags + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != sk.epoch) {
                        if (++spins > kStreamKSpinLimit) {
                            fail = 1;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
                    }
                    s_fail = fail;
                }
                __syncthreads();
                const bool fail = s_fail != 0;
                const uint32_t sbase = uint32_t(w) * uint32_t(BM * BN * 4);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j) {
                        const f32x4 p = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                       prsrc, int(sbase + uint32_t(((i * TN + j) * NT + tid) * 16)), 0, kDeviceScope));
                        acc[i][j] = fail ? f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                                                 __builtin_nanf("")}
                                         : acc[i][j] + p;
                    }
                __syncthreads();   // s_fail is rewritten for the next piece
            }
        }
        store_tile<T, BM, BN, WM, WN, TM, TN, NHWC_OUT>(g, acc, m0, n0, wm, wn, lane);
    }
}

}  // namespace convlower
