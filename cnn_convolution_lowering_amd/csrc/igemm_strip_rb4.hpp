// Unrolled-tap strip kernel on 16x16x32 MFMAs with the filter shared through
// LDS (16-bit NHWC, unit horizontal dilation, S a template value).
//
// conv_strip_rb3_kernel's contraction, strips and pixel layout, but the
// filter fragments of a tap are brought in once per workgroup: with one
// column of waves every wave needs the same output-channel fragments, and in
// the register form each wave fetched all of them.  Here the waves split a
// tap's fragments between them and load them with LDS-DMA into a ring of
// FD+1 LDS slots, FD taps ahead; every wave reads its fragments of the next
// tap from LDS while the current tap's MFMAs run.  One barrier per tap:
// before it each wave waits for its own loads of the next tap's slot and for
// its own LDS reads of two taps back, so that past it that slot is complete
// for every wave and the slot read two taps back is free to load again (the
// ring's extra slot lets the reads of the tap just ended stay in flight).
// Output-channel fragments are the outer loop of a tap, so each filter
// register is reloaded as soon as its column of MFMAs is done and only the
// pixel fragments are double-buffered.
#pragma once

#include "igemm_strip_rb3.hpp"

namespace convlower {

// Strip loads a wave issues at the taps p0 .. p1-1 of a strip (negative: the
// previous strip's taps S+p), NLA of them spread PER a tap over the first
// DSTEPS taps.
constexpr int rb4_strip_loads_between(int p0, int p1, int S, int DSTEPS, int PER, int NLA) {
    int c = 0;
    for (int p = p0; p < p1; ++p) {
        const int q = p < 0 ? p + S : p;
        const int n = q < DSTEPS ? NLA - q * PER : 0;
        c += n < 0 ? 0 : (n > PER ? PER : n);
    }
    return c;
}

// FD: how many taps ahead the filter slots are loaded (the ring holds FD+1).
// DIRECT: the filter is read as the caller's KRSC rows (a fragment lane's 8
// channels are 16 contiguous bytes of one row) instead of the 16x16x32
// fragment-order copy, so the layer needs no packing pass.
template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int S, int FD, bool DIRECT>
__global__ void __launch_bounds__(64 * WGM * WGN, (strip_rb_min_blocks<BM, BN, WGM, WGN>()))
    conv_strip_rb4_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = NT / 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int NM = TM * TN;
    constexpr int NF = BN / 16;                 // filter fragments of a tap for the workgroup
    constexpr int FPW = NF / NW;                // of them, loaded by each wave
    constexpr int NS = FD + 1;                  // filter slots
    constexpr int SLOT = NF * 1024;             // bytes per slot
    constexpr int BUF = STRIP * 16;             // bytes per strip buffer
    using ASrc = PaddedStripOr<T, NT, STRIP>;
    constexpr int NLA = ASrc::NL;
    constexpr int DSTEPS = S > 3 ? 3 : S - 1;                   // steps the next strip's loads are spread over
    constexpr int PER = (NLA + DSTEPS - 1) / DSTEPS;             // strip loads per such step
    static_assert(sizeof(T) == 2, "16-bit storage");
    static_assert(STRIP % NT == 0 && WM % 16 == 0 && WN % 16 == 0 && NF % NW == 0 && FPW >= 1, "tile shape");
    static_assert(FD >= 2 && FD <= S && NS == FD + 1 && DSTEPS >= 1 && DSTEPS < S, "prefetch distances");
    static_assert(TM >= 2 && FPW + TM + PER <= TN * (TM - 1), "one memory operation per MFMA");
    static_assert(NLA + FD * FPW < 64, "vmcnt range");
    static_assert(S * kStripRb2RowBytes < 65536 && NS * SLOT <= 65536, "offsets fit an instruction offset");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF + NS * SLOT];

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

    // B fragments (pixels) as in the register form.
    const int pl = 2 * (lane & 7) + ((lane >> 3) & 1);
    uint32_t aoff[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 16 + pl;
        int32_t sr = 0;
        if (m < g.M) {
            const int32_t gr = int32_t(m / g.Q);
            sr = (gr - g0) * w_used + (int32_t(m) - gr * g.Q) * g.sw;
        }
        aoff[i] = uint32_t(sr * kStripRb2RowBytes + (lane >> 4) * 16);
    }

    // Packed filter (pack_filter_frag16_kernel): fragment (nb, kk) at
    // ((nb*KK + kk)*64 + lane)*16 bytes.  This wave loads fragments
    // f = wave*FPW + q of each tap (output-channel block n0/16 + f, the
    // copy's last block again past it: its outputs are never stored), the
    // whole offset in the range-checked part.
    //
    // DIRECT: lane l of fragment (nb, kk) reads 16 bytes of KRSC row
    // nb*16 + l%16 at element kk*32 + 8*(l/16); rows past K lie past the
    // filter's K*Kc elements (below 2^31 bytes, checked on the host) and read
    // as zero.  Tap positions below are in bytes of the packed copy (1 KiB per
    // 32-deep step) or of a KRSC row (64 bytes per step).
    const int KK = g.Kc / 32;
    const int NBt = (g.K + 15) / 16;
    const i32x4 frsrc = DIRECT ? make_rsrc(g.b, uint32_t(int64_t(g.K) * g.Kc * int(sizeof(T))))
                               : make_rsrc(g.b, uint32_t(int64_t(NBt) * KK * 1024));
    uint32_t flane[FPW];
#pragma unroll
    for (int q = 0; q < FPW; ++q) {
        const int nb = min(n0 / 16 + wave * FPW + q, NBt - 1);
        flane[q] = DIRECT ? uint32_t((int64_t(nb * 16 + (lane & 15)) * g.Kc + (lane >> 4) * 8) * int(sizeof(T)))
                          : uint32_t((int64_t(nb) * KK * 64 + lane) * 16);
    }
    constexpr int FB = DIRECT ? 2 : 32;                                          // bytes per filter element position
    const int tap_bytes = g.C * FB;                                               // one tap of the filter rows
    auto kbase = [&](int r, int cb) { return (r * S * g.C + cb * 32) * FB; };    // tap 0 of strip (r, cb)

    const uint32_t lds0 = lds_offset(smem);
    const uint32_t slots0 = lds0 + uint32_t(2 * BUF);
    auto strip_load = [&](int buf, int j, int r, int cb, bool on) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, r, cb, on), lds0 + uint32_t(buf * BUF) + uint32_t((j * NT + wave * 64) * 16));
    };
    // this wave's share of the filter of the tap at byte offset kpos, into
    // slot sl
    auto filter_load = [&](int q, int kpos, int sl) __attribute__((always_inline)) {
        dma16(frsrc, flane[q] + uint32_t(kpos), slots0 + uint32_t(sl * SLOT + (wave * FPW + q) * 1024));
    };
    auto lds16 = [&](uint32_t byte_off) __attribute__((always_inline)) { return load16(smem + byte_off); };
    // the lane's fragment j of a slot: byte offset from smem
    const uint32_t fb_lane = uint32_t(2 * BUF + wn * TN * 1024 + lane * 16);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int CB = g.C / 32;
    const int nstrips = g.R * CB;

    // Prologue: strip 0 into buffer 0, the filter of taps 0 .. FD-1 of strip
    // 0 (FD <= S) into slots 0 .. FD-1, then the fragments of tap 0.
#pragma unroll
    for (int j = 0; j < NLA; ++j) strip_load(0, j, 0, 0, true);
#pragma unroll
    for (int d = 0; d < FD; ++d)
#pragma unroll
        for (int q = 0; q < FPW; ++q) filter_load(q, kbase(0, 0) + d * tap_bytes, d);
    wait_vmcnt<0>();
    lds_barrier();
    u32x4 fa[TM], fan[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = lds16(aoff[i]);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = lds16(fb_lane + uint32_t(j * 1024));

    // Slot of tap t + 1 (read during tap t) and of tap t + FD (loaded during
    // tap t), as the taps go by.
    int sl_rd = 1, sl_ld = FD;

    auto strip = [&](int r, int cb, int r1, int cb1, int buf, bool has_next) __attribute__((always_inline)) {
        const int kb = kbase(r, cb);
        const int kb1 = has_next ? kbase(r1, cb1) : 0;
        uint32_t abase[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) abase[i] = aoff[i] + uint32_t(buf * BUF);
        static_for<S>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            // filter of tap s + FD: this strip or the next; past the last
            // strip, position 0 again into a slot no MFMA reads
            constexpr bool nxt = s + FD >= S;
            constexpr int sb = nxt ? s + FD - S : s + FD;
            const int kfd = nxt ? (has_next ? kb1 + sb * tap_bytes : 0) : kb + sb * tap_bytes;
            // Before the barrier: this wave's loads of tap t+1's slot (issued
            // at tap t+1-FD, first in that tap) have landed -- younger are the
            // filter loads of the FD-2 taps in between and the strip loads
            // of taps t+1-FD .. t-1 -- and, at the strip's last tap, its loads
            // of the next strip (younger: the filter loads of the taps since).
            // Its LDS reads of tap t-2 and before are done (younger: the
            // TM + TN reads of tap t-1): the slot loaded from here on was last
            // read in tap t-2, and so was the strip buffer the next strip's
            // loads go to.
            constexpr int W_FILT = FPW * (FD - 2) + rb4_strip_loads_between(s + 1 - FD, s, S, DSTEPS, PER, NLA);
            constexpr int W_STRIP = FPW * (S - 1 - DSTEPS);
            constexpr int WAIT = s == S - 1 ? (W_FILT < W_STRIP ? W_FILT : W_STRIP) : W_FILT;
            constexpr int LGKM = TM + TN < 15 ? TM + TN : 15;
            static_assert(WAIT >= 0 && WAIT < 64, "vmcnt range");
            wait_vmcnt<WAIT>();
            __builtin_amdgcn_s_waitcnt(0xC07F | (LGKM << 8));   // lgkmcnt(LGKM)
            lds_barrier();
            const uint32_t fb_next = fb_lane + uint32_t(sl_rd * SLOT);
            // MFMAs output-channel fragment by fragment (j outer); after
            // fragment j's last, its register takes the next tap's fragment j
            // from the next slot.  On the other slots: this wave's share of
            // the filter of tap t+FD, the next tap's pixel fragments into
            // fan, and in the first DSTEPS taps the next strip's loads.
            static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int j = idx / TM, i = idx % TM;
                acc[i][j] = Mfma<T>::run(fb[j], fa[i], acc[i][j]);
                constexpr int q = idx / TM * (TM - 1) + idx % TM;   // q-th MFMA without a filter read
                if constexpr (i == TM - 1) {
                    fb[j] = lds16(fb_next + uint32_t(j * 1024));
                } else if constexpr (q < FPW) {
                    filter_load(q, kfd, sl_ld);
                } else if constexpr (q < FPW + TM) {
                    constexpr int ii = q - FPW;
                    if constexpr (s + 1 < S)
                        fan[ii] = lds16(abase[ii] + uint32_t((s + 1) * kStripRb2RowBytes));
                    else
                        fan[ii] = lds16(aoff[ii] + uint32_t((buf ^ 1) * BUF));
                } else if constexpr (s < DSTEPS) {
                    constexpr int p = q - FPW - TM;
                    if constexpr (p < PER && s * PER + p < NLA) strip_load(buf ^ 1, s * PER + p, r1, cb1, has_next);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = fan[i];
            sl_rd = sl_rd + 1 == NS ? 0 : sl_rd + 1;
            sl_ld = sl_ld + 1 == NS ? 0 : sl_ld + 1;
        });
    };

    int r = 0, cb = 0;
    for (int j = 0; j < nstrips; ++j) {
        int r1 = r, cb1 = cb + 1;
        if (cb1 == CB) {
            cb1 = 0;
            ++r1;
        }
        strip(r, cb, r1, cb1, j & 1, j + 1 < nstrips);
        r = r1;
        cb = cb1;
    }
    // loads past the last strip still write this workgroup's LDS
    wait_vmcnt<0>();

    // Fused epilogue as in the register form.
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    const int kl = 4 * (lane >> 4);
    float bv[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int k = n0 + wn * WN + j * 16 + kl;
        if (bias && (g.K & 3) == 0 && k + 3 < g.K) {
            union {
                u32x2 u;
                T e[4];
            } pk;
            pk.u = *reinterpret_cast<const u32x2*>(bias + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[j][e] = to_f32(pk.e[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[j][e] = (bias && k + e < g.K) ? to_f32(bias[k + e]) : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 16 + pl;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int k = n0 + wn * WN + j * 16 + kl;
            T* dst = y + m * g.K + k;
            if (k + 3 < g.K && (g.K & 3) == 0) {
                union {
                    u32x2 u;
                    T e[4];
                } pk;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(acc[i][j][e] + bv[j][e]);
                *reinterpret_cast<u32x2*>(dst) = pk.u;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (k + e < g.K) dst[e] = from_f32<T>(acc[i][j][e] + bv[j][e]);
            }
        }
    }
}

}  // namespace convlower
