// Register-streamed strip kernel with the taps of a filter row unrolled at
// compile time (16-bit NHWC, unit horizontal dilation, S a template value).
//
// The same contraction as conv_strip_rb_kernel -- per filter row r and block
// of 32 channels, the input rows under the tile's output rows copied once
// into LDS and read by all S taps ("Enabling Memory-efficient Im2win
// Convolution with Multi-precision Support on GPU CUDA and Tensor Cores",
// abstract), the filter streamed into registers from its fragment-order copy
// -- laid out so that the work around the MFMAs is nearly free.  Measured on
// the general kernel, the address arithmetic, position bookkeeping and
// branches of a step cost about as much as its 32 MFMAs and did not overlap
// them.  Here:
//   - strip rows are padded to 80 bytes (four 16-byte chunks and a zero
//     slot), and the 32 pixels of an MFMA fragment are dealt to lanes with
//     lane bits 3 and 4 exchanged, so the 16 lanes the LDS serves together
//     read 16 consecutive rows: 16 different 4-bank groups, no conflict,
//     without any swizzle.  A lane's A address is then a fixed register plus
//     the tap times 80 bytes (an instruction offset), and the second 16-deep
//     half two chunks further (another offset);
//   - the S taps of a strip are one unrolled body, so the filter position of
//     a step is the strip's base plus a compile-time multiple of the tap
//     stride (scalar), and the register ring of filter fragments is indexed
//     at compile time (one body per ring phase);
//   - the next strip's loads go out over the first steps of the current one
//     (so they are in flight while it computes), and the one wait and barrier
//     of a strip sits before the second half of its last step.
#pragma once

#include "igemm_strip_rb.hpp"

namespace convlower {

// The input strip of one (r, channel block) in padded rows: 16-byte slot
// q = 5*row + chunk (chunk 4 is padding, loaded as zeros).  Row
// t*W_used + col holds the input row under output row g0 + t, column col.
template <typename T, int NT, int STRIP>
struct PaddedStripSrc {
    static constexpr int NL = STRIP / NT;
    int32_t base[NL];   // bytes to x[n][p*sh - ph][w][chunk*8] (r = 0, block 0)
    int32_t hrow[NL];   // p*sh - ph, or far out of range for padding, rows past the strip and columns outside the image
    i32x4 rsrc;

    __device__ __forceinline__ void init(const GemmArgs& g, int32_t g0, int32_t t_rows, int32_t w_used, int tid) {
        const int64_t x_bytes = (g.M / g.PQ) * int64_t(g.H) * g.W * g.C * int64_t(sizeof(T));
        rsrc = make_rsrc(g.a, uint32_t(x_bytes < int64_t(0x7fffffff) ? x_bytes : int64_t(0x7fffffff)));
        const int32_t P = g.PQ / g.Q;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int slot = j * NT + tid;
            const int row = slot / 5;
            const int chunk = slot - row * 5;
            const int t = row / w_used;
            const int col = row - t * w_used;
            const int32_t gr = g0 + (t < t_rows ? t : 0);
            const int32_t n = gr / P;
            const int32_t p = gr - n * P;
            const int32_t w = col - g.pw;
            const int32_t hv = p * g.sh - g.ph;
            const bool ok = chunk < 4 && t < t_rows && unsigned(w) < unsigned(g.W);
            base[j] = ((n * g.H + hv) * g.W + (ok ? w : 0)) * g.C * int32_t(sizeof(T)) + (chunk & 3) * 16;
            hrow[j] = ok ? hv : -(1 << 28);
        }
    }
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j, int r, int cb) const {
        const int32_t h = hrow[j] + r * g.dh;
        const int32_t o = base[j] + ((r * g.dh * g.W) * g.C + cb * 32) * int32_t(sizeof(T));
        return unsigned(h) < unsigned(g.H) ? uint32_t(o) : kOutOfRange;
    }
};

constexpr int kStripRb2RowBytes = 80;

// DB_MAX: how many steps ahead the filter fragments are loaded, at most
// (one strip ahead at most: S - 1 for narrow filters).
template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int S, int DB_MAX>
__global__ void __launch_bounds__(64 * WGM * WGN, (strip_rb_min_blocks<BM, BN, WGM, WGN>()))
    conv_strip_rb2_kernel(GemmArgs g) {
    constexpr int DB = DB_MAX < S ? DB_MAX : S - 1;
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int NM = TM * TN;
    constexpr int NR = DB + 1;            // filter register ring
    constexpr int BUF = STRIP * 16;       // bytes per strip buffer
    using ASrc = PaddedStripSrc<T, NT, STRIP>;
    constexpr int NLA = ASrc::NL;
    constexpr int DSTEPS = S > 3 ? 3 : S - 1;                   // steps the next strip's loads are spread over
    constexpr int PER = (NLA + DSTEPS - 1) / DSTEPS;             // strip loads per such step
    constexpr int WAIT = 2 * TN * (S - DSTEPS) < 63 ? 2 * TN * (S - DSTEPS) : 63;
    static_assert(sizeof(T) == 2, "16-bit storage");
    static_assert(STRIP % NT == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(DB >= 1 && DB < S && DSTEPS >= 1 && DSTEPS < S, "prefetch distances");
    static_assert((S - 1) * kStripRb2RowBytes + 32 < 4096, "tap offsets fit an instruction offset");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int tile_n = tile - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    const int32_t w_used = (g.Q - 1) * g.sw + (S - 1) + 1;
    const int64_t m_last = (m0 + BM < g.M ? m0 + BM : g.M) - 1;
    const int32_t g0 = int32_t(m0 / g.Q);
    const int32_t t_rows = int32_t(m_last / g.Q) - g0 + 1;

    ASrc la;
    la.init(g, g0, t_rows, w_used, tid);

    // The lane's pixel within a 32-pixel fragment: lane bits 3 and 4
    // exchanged, so lanes {0-7, 16-23} (and each other group of 16 the LDS
    // serves in one cycle) take 16 consecutive pixels.  The MFMA's B columns
    // and its output columns follow the same lane order.
    const int pl = (lane & 7) | ((lane & 8) << 1) | ((lane & 16) >> 1);
    uint32_t aoff[TM];   // byte offset in a strip buffer: the lane's row at tap 0, chunk lane/32
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 32 + pl;
        int32_t sr = 0;
        if (m < g.M) {
            const int32_t gr = int32_t(m / g.Q);
            sr = (gr - g0) * w_used + (int32_t(m) - gr * g.Q) * g.sw;
        }
        aoff[i] = uint32_t(sr * kStripRb2RowBytes + (lane >> 5) * 16);
    }

    // Packed filter: fragment (nb, kk) at ((nb*KK + kk)*64 + lane)*16 bytes;
    // contraction position pos (a multiple of 16) is kk = pos/16, i.e.
    // pos*64 bytes into a block's run.
    const int KK = g.Kc / 16;
    const int NBt = (g.K + 31) / 32;
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.b), 0, int(int64_t(NBt) * KK * 1024), 0x00020000);
    const int nb0 = (n0 + wn * WN) / 32;
    uint32_t bfrag[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int nb = nb0 + j < NBt ? nb0 + j : NBt - 1;
        bfrag[j] = uint32_t((int64_t(nb) * KK * 64 + lane) * 16);
    }
    const int tap_bytes = g.C * 64;                                      // one tap of the filter rows
    auto kbase = [&](int r, int cb) { return (r * S * g.C + cb * 32) * 64; };   // tap 0 of strip (r, cb)

    const uint32_t lds0 = lds_offset(smem);
    auto strip_load = [&](int buf, int j, int r, int cb) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, r, cb), lds0 + uint32_t(buf * BUF) + uint32_t((j * NT + wave * 64) * 16));
    };
    auto lds16 = [&](uint32_t byte_off) __attribute__((always_inline)) { return load16(smem + byte_off); };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int CB = g.C / 32;
    const int nstrips = g.R * CB;

    // Prologue: strip 0 into buffer 0, the filter fragments of taps 0 .. DB-1
    // of strip 0, then the A fragments of its first half-step.
#pragma unroll
    for (int j = 0; j < NLA; ++j) strip_load(0, j, 0, 0);
    u32x4 fb[NR][2][TN];
    static_for<DB>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[d][h][j] = buffer_load16(brsrc, bfrag[j], d * tap_bytes + h * 1024);
    });
    wait_vmcnt<0>();
    lds_barrier();
    u32x4 fa0[TM], fa1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa0[i] = lds16(aoff[i]);

    // One strip: S steps of two 16-deep halves.  Ring phase PH: the filter
    // fragments of tap s are in set (PH + s) % NR.
    auto strip = [&](auto phc, int r, int cb, int r1, int cb1, int buf, bool has_next) __attribute__((always_inline)) {
        constexpr int PH = decltype(phc)::value;
        const int kb = kbase(r, cb);
        const int kb1 = has_next ? kbase(r1, cb1) : 0;
        uint32_t abase[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) abase[i] = aoff[i] + uint32_t(buf * BUF);
        static_for<S>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            constexpr int RC = (PH + s) % NR;
            constexpr int RL = (PH + s + DB) % NR;
            // filter fragments of tap s + DB: this strip or the next; past
            // the last strip, position 0 again into a set nobody reads (the
            // loads stay unconditional, so the compiler's count is exact)
            constexpr bool nxt = s + DB >= S;
            constexpr int sb = nxt ? s + DB - S : s + DB;
            const int kbb = nxt ? (has_next ? kb1 + sb * tap_bytes : 0) : kb + sb * tap_bytes;
            // ---- half 0: A fragments of half 1, filter half 0 of tap s+DB,
            // the next strip's loads (first DSTEPS steps)
            static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int i = idx / TN, j = idx % TN;
                acc[i][j] = Mfma32<T>::run(fb[RC][0][j], fa0[i], acc[i][j]);
                if constexpr (idx < TM) {
                    fa1[idx] = lds16(abase[idx] + uint32_t(s * kStripRb2RowBytes + 32));
                } else if constexpr (idx < TM + TN) {
                    fb[RL][0][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kbb);
                } else if constexpr (s < DSTEPS && idx - TM - TN < PER && s * PER + idx - TM - TN < NLA) {
                    if (has_next) strip_load(buf ^ 1, s * PER + idx - TM - TN, r1, cb1);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            static_for<(TM + TN + PER > NM ? TM + TN + PER - NM : 0)>([&](auto rc) __attribute__((always_inline)) {
                constexpr int idx = NM + decltype(rc)::value;
                if constexpr (idx < TM) {
                    fa1[idx] = lds16(abase[idx] + uint32_t(s * kStripRb2RowBytes + 32));
                } else if constexpr (idx < TM + TN) {
                    fb[RL][0][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kbb);
                } else if constexpr (s < DSTEPS && s * PER + idx - TM - TN < NLA) {
                    if (has_next) strip_load(buf ^ 1, s * PER + idx - TM - TN, r1, cb1);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
            // ---- half 1: A fragments of the next step (at the strip's last
            // step, of the next strip, after its loads landed for every wave
            // and every wave finished reading this buffer), filter half 1
            if constexpr (s == S - 1) {
                if (has_next) {
                    // loads issued after this wave's last strip load: its filter
                    // loads of the steps since (more in flight than the count's
                    // range only makes the wait stricter)
                    wait_vmcnt<WAIT>();
                    asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
                    lds_barrier();
                }
            }
            static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int i = idx / TN, j = idx % TN;
                acc[i][j] = Mfma32<T>::run(fb[RC][1][j], fa1[i], acc[i][j]);
                if constexpr (idx < TM) {
                    if constexpr (s + 1 < S) {
                        fa0[idx] = lds16(abase[idx] + uint32_t((s + 1) * kStripRb2RowBytes));
                    } else {
                        if (has_next) fa0[idx] = lds16(aoff[idx] + uint32_t((buf ^ 1) * BUF));
                    }
                } else if constexpr (idx < TM + TN) {
                    fb[RL][1][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kbb + 1024);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            static_for<(TM + TN > NM ? TM + TN - NM : 0)>([&](auto rc) __attribute__((always_inline)) {
                constexpr int idx = NM + decltype(rc)::value;
                if constexpr (idx < TM) {
                    if constexpr (s + 1 < S) {
                        fa0[idx] = lds16(abase[idx] + uint32_t((s + 1) * kStripRb2RowBytes));
                    } else {
                        if (has_next) fa0[idx] = lds16(aoff[idx] + uint32_t((buf ^ 1) * BUF));
                    }
                } else {
                    fb[RL][1][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kbb + 1024);
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    int r = 0, cb = 0, ph = 0;
    for (int j = 0; j < nstrips; ++j) {
        int r1 = r, cb1 = cb + 1;
        if (cb1 == CB) {
            cb1 = 0;
            ++r1;
        }
        const bool has_next = j + 1 < nstrips;
        const int buf = j & 1;
        static_for<NR>([&](auto pc) __attribute__((always_inline)) {
            if (ph == decltype(pc)::value) strip(pc, r, cb, r1, cb1, buf, has_next);
        });
        ph = (ph + S) % NR;
        r = r1;
        cb = cb1;
    }

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
        const int64_t m = m0 + wm * WM + i * 32 + pl;
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
