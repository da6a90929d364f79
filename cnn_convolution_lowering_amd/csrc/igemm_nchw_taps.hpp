// fp32 NCHW tap-expanded implicit contraction: the window elements of a
// tile's pixels staged in LDS one (channel, tap) plane at a time, for the
// strided encoder layers (any padding, stride and dilation; C a multiple of
// 16; filter widths 2 and 3 compiled).
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract) and the im2col lowering of "A
// Simple and Efficient Implementation of im2col in Convolution Neural
// Networks" (Section 2): the contraction of output pixel m over (c, r, s) reads
// x[n][c][p*sh - ph + r*dh][q*sw - pw + s*dw].  For filter row r and a block
// of 16 input channels the workgroup gathers, for every one of its BM
// pixels, the element of each channel and tap of that row into plane
// (c, s) -- a row of the im2col matrix restricted to the tile -- with 4-byte
// LDS-DMA loads (zero outside the image and past the last pixel).  A step
// (16 channels of one tap) then reads 16 consecutive words of a plane per
// lane group: the planes of the four lane groups start 16 banks apart
// (pitch nchw_taps_pitch), so the reads are free of bank conflicts for any
// stride, where a strip of input rows read at stride sw puts every lane of a
// stride-2 layer on even banks.
//
// Contraction order, filter fragments and MFMA (v_mfma_f32_16x16x4_f32) as
// the NCHW strip kernel: strip (cb, r) after strip, one step per tap, lane
// group gq taking channels 4*gq .. 4*gq+3 (pack_filter_frag_f32_kernel).
// The filter is streamed into registers (NBUF-1)*S - 1 steps ahead, and the
// strips through a ring of NBUF LDS buffers, strip i+NBUF loaded as soon as
// strip i's buffer is free.  Every step issues the same loads whatever the
// strip, and the taps are compiled, so that the compiler's vmcnt waits for
// the filter registers are exact and never hold a wave on a strip still in
// flight.
#pragma once

#include "dispatch.hpp"
#include "igemm_nchw.hpp"
#include "igemm_strip_rb.hpp"

namespace convlower {

// Words from one (channel, tap) plane to the next (nchw_taps_plane): the
// first BMP >= BM with 4*S*BMP an odd multiple of 16 modulo 64, so that lane
// group gq, which reads channel 4*gq + e, starts 16*gq*odd banks from group
// 0 (BM where no such pitch exists, S a multiple of 8).
template <int BM, int S>
constexpr int nchw_taps_pitch() { return nchw_taps_plane(BM, S); }

template <int BM, int S>
constexpr int nchw_taps_buffer_bytes() { return 16 * S * nchw_taps_pitch<BM, S>() * 4; }

template <int BM, int BN, int WGM, int WGN, int NBUF, int S>
__global__ void __launch_bounds__(64 * WGM * WGN, 2) conv_nchw_f32_taps_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = NT / 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int BMP = nchw_taps_pitch<BM, S>();
    constexpr int BUFB = nchw_taps_buffer_bytes<BM, S>();   // bytes per strip buffer
    constexpr int HALVES = BM / 64;                           // 64-pixel runs per plane
    constexpr int NL = 16 * S * HALVES / NW;                  // 4-byte loads per lane per strip
    constexpr int NR = (NBUF - 1) * S;                        // filter ring: DB = NR - 1 steps ahead
    constexpr int DB = NR - 1;
    constexpr int NM = 4 * TM * TN;
    static_assert(NT == 256 && BM % 64 == 0 && NW % HALVES == 0 && (16 * HALVES) % NW == 0 && WM % 16 == 0 &&
                      WN % 16 == 0 && NBUF >= 2 && S >= 2,
                  "tile shape");
    static_assert(TM + TN + NL <= NM, "one load per MFMA");
    // At the last step of strip i, before its own loads: the loads issued
    // after strip i+1's (issued at the last step of strip i+1-NBUF) are the
    // NBUF-2 strips in between (S*TN filter and NL strip loads each) and the
    // filter loads of strip i's first S-1 steps.
    constexpr int WAIT = (NBUF - 2) * (S * TN + NL) + (S - 1) * TN;
    // (Loads in flight at once: at most the NBUF-1 strips after the one
    // waited for and the filter ring; the prologue waits where it has more.)
    static_assert(WAIT < 64 && (NBUF - 1) * NL + NR * TN < 64 && NL + DB * TN < 64 &&
                      (NBUF != 2 || 2 * NL + DB * TN < 64),
                  "vmcnt range");

    constexpr int OP = BM + 4;   // pitch of the channel-major output tile in the epilogue
    constexpr int SMEM_B = NBUF * BUFB > BN * OP * 4 ? NBUF * BUFB : BN * OP * 4;
    __shared__ __attribute__((aligned(16))) float smem[SMEM_B / 4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;

    // x has fewer than 2^29 elements, so every element offset fits 32 bits.
    const int32_t M = int32_t(g.M);
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int n0 = (tile - tile_m * g.tiles_n) * BN;
    const int32_t m0 = tile_m * BM;

    // This lane's gathered pixel (the same for all of its loads: wave w
    // fills the 64-pixel run w % HALVES of planes (w / HALVES)*NL .. +NL-1,
    // instruction j plane (w / HALVES)*NL + j, i.e. channel
    // (w / HALVES)*NL/S + j/S and tap j % S) and its offset in x for
    // (c, r, s) = (0, 0, 0).
    const int32_t HW = g.H * g.W;
    const int half = wave % HALVES;
    const int cgrp = wave / HALVES;
    const int32_t pm = m0 + half * 64 + lane;
    int32_t pix_off, h_base, w_base;
    {
        const int32_t mm = pm < M ? pm : 0;
        const int32_t n = mm / g.PQ, pq = mm - n * g.PQ;
        const int32_t p = pq / g.Q, q = pq - p * g.Q;
        w_base = q * g.sw - g.pw;
        pix_off = (n * g.C * g.H + p * g.sh - g.ph) * g.W + w_base;
        h_base = pm < M ? p * g.sh - g.ph : -(1 << 28);   // far out of range past the last pixel
    }
    // kOutOfRange where tap s of this lane's pixel falls outside the image
    // columns (ORed into the offsets: the load then reads zero).
    uint32_t w_bad[S];
#pragma unroll
    for (int s = 0; s < S; ++s) w_bad[s] = unsigned(w_base + s * g.dw) < unsigned(g.W) ? 0u : kOutOfRange;
    const int n_img = M / g.PQ;
    const i32x4 xrsrc = make_rsrc(g.a, uint32_t(n_img * g.C * HW * 4));
    const uint32_t lds0 = lds_offset(smem);

    // Load j of the strip being loaded (ld_off: this lane's offset in x of
    // its channel 0, tap 0; ld_bad: kOutOfRange where its filter row falls
    // outside the image or the strip is past the last, whose zeros land in a
    // buffer nobody reads again) into buffer buf.  Valid offsets are below
    // 2^31, so ORing kOutOfRange in is what makes the load read zero.
    int32_t ld_off = 0;
    uint32_t ld_bad = 0;
    auto strip_load = [&](int buf, auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        constexpr int c = j / S, s = j % S;
        const int32_t uni = (cgrp * (NL / S) + c) * HW + s * g.dw;
        dma4(xrsrc, (uint32_t(ld_off + uni) * 4u) | ld_bad | w_bad[s],
             lds0 + uint32_t(buf * BUFB) + uint32_t(((cgrp * NL + j) * BMP + half * 64) * 4));
    };

    // Packed filter: fragment (nb, kk) at ((nb*KK + kk)*64 + lane)*16 bytes.
    const int KK = g.Kc / 16;
    const int NBt = (g.K + 15) / 16;
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.b), 0, int(int64_t(NBt) * KK * 1024), 0x00020000);
    uint32_t bfrag[TN];
    float bias_v[TN];
    const float* __restrict__ bias = static_cast<const float*>(g.bias);
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int nb = (n0 + wn * WN) / 16 + j;
        bfrag[j] = uint32_t((int64_t(nb < NBt ? nb : NBt - 1) * KK * 64 + lane) * 16);
        const int n = n0 + wn * WN + j * 16 + (lane & 15);
        bias_v[j] = (bias && n < g.K) ? bias[n] : 0.f;
    }

    // A fragment i of tap s from buffer buf: lane (gq, l16) element e is
    // plane (4*gq + e, s) at pixel wm*WM + i*16 + l16.
    const int gq = lane >> 4;
    const float* const sl = smem + (4 * gq * S) * BMP + wm * WM + (lane & 15);
    auto read_a = [&](u32x4& fa, int i, int buf, int s) __attribute__((always_inline)) {
        const float* sa = sl + buf * (BUFB / 4) + s * BMP + i * 16;
        fa = u32x4{__float_as_uint(sa[0]), __float_as_uint(sa[S * BMP]), __float_as_uint(sa[2 * S * BMP]),
                   __float_as_uint(sa[3 * S * BMP])};
    };

    const int CBN = g.C / 16;
    const int nstrips = g.R * CBN;
    const int nsteps = nstrips * S;

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The next strip to load: (nr, ncb), index nld.
    int nld = 0, nr = 0, ncb = 0;
    auto set_load = [&]() __attribute__((always_inline)) {
        ld_off = pix_off + ncb * 16 * HW + nr * g.dh * g.W;
        ld_bad = (unsigned(h_base + nr * g.dh) < unsigned(g.H) ? 0u : kOutOfRange) |
                 (nld < nstrips ? 0u : kOutOfRange);
    };
    auto advance = [&]() __attribute__((always_inline)) {
        ++nld;
        if (++nr == g.R) {
            nr = 0;
            ++ncb;
        }
        set_load();
    };
    set_load();

    // Prologue: strips 0 .. NBUF-1 into buffers 0 .. NBUF-1, filter
    // fragments of steps 0 .. DB-1 (with at most 63 loads in flight).  Two
    // buffers: strip 0, the filter, then strip 1, and the steps start once
    // strip 0 and the filter have landed (strip 1 is waited for at the end of
    // strip 0, with the same count as every later strip).  More buffers: all
    // of it landed first, so that those counts hold from the first strip on.
    u32x4 fb[NR][TN];
    auto prologue_filter = [&]() __attribute__((always_inline)) {
        static_for<DB>([&](auto dc) __attribute__((always_inline)) {
            constexpr int d = decltype(dc)::value;
            const int kp = d < nsteps ? d : 0;
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[d][j] = buffer_load16(brsrc, bfrag[j], kp * 1024);
        });
    };
    if constexpr (NBUF == 2) {
        static_for<NL>([&](auto jc) __attribute__((always_inline)) { strip_load(0, jc); });
        advance();
        prologue_filter();
        static_for<NL>([&](auto jc) __attribute__((always_inline)) { strip_load(1, jc); });
        advance();
        wait_vmcnt<NL>();
    } else {
        static_for<NBUF>([&](auto sbc) __attribute__((always_inline)) {
            constexpr int sb = decltype(sbc)::value;
            if constexpr ((sb + 1) * NL > 63) wait_vmcnt<63 - NL>();
            static_for<NL>([&](auto jc) __attribute__((always_inline)) { strip_load(sb, jc); });
            advance();
        });
        if constexpr (NBUF * NL + DB * TN > 63) wait_vmcnt<63 - DB * TN>();
        prologue_filter();
        wait_vmcnt<0>();
    }
    lds_barrier();

    u32x4 fa0[TM], fa1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a(fa0[i], i, 0, 0);

    // Strip i in buffer buf with filter-ring base RB: S steps.  Step s runs
    // its MFMAs on fa0 and, one per MFMA, reads the A fragments of the next
    // step (tap s+1, or tap 0 of strip i+1 in the next buffer) into fa1,
    // loads the filter fragments of step k+DB, and at the last step loads
    // strip i+NBUF into this strip's buffer.  The last step first waits for
    // strip i+1 (this wave's loads, then the barrier for every wave's) and
    // for this wave's reads of the strip: past the barrier no wave reads it.
    auto strip = [&](int i, int buf, auto rbc) __attribute__((always_inline)) {
        constexpr int RB = decltype(rbc)::value;
        const int buf_n = buf + 1 == NBUF ? 0 : buf + 1;
        static_for<S>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            constexpr int RC = RB + s;
            constexpr int RL = (RC + DB) % NR;
            constexpr bool LAST = s == S - 1;
            if constexpr (LAST) {
                wait_vmcnt<WAIT>();
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                lds_barrier();
            }
            const int k = i * S + s;
            const int kp = k + DB < nsteps ? k + DB : 0;
            static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int e = idx / (TM * TN), ii = (idx / TN) % TM, jj = idx % TN;
                const uint32_t av = fa0[ii][e], bv = fb[RC][jj][e];
                acc[ii][jj] =
                    __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av), __uint_as_float(bv), acc[ii][jj], 0, 0, 0);
                if constexpr (idx < TM) {
                    if constexpr (LAST)
                        read_a(fa1[idx], idx, buf_n, 0);
                    else
                        read_a(fa1[idx], idx, buf, s + 1);
                } else if constexpr (idx < TM + TN) {
                    fb[RL][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kp * 1024);
                } else if constexpr (LAST && idx < TM + TN + NL) {
                    strip_load(buf, std::integral_constant<int, idx - TM - TN>{});
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            if constexpr (LAST) advance();
#pragma unroll
            for (int ii = 0; ii < TM; ++ii) fa0[ii] = fa1[ii];
        });
    };

    // NBUF-1 strips per pass, so that the filter ring starts each pass at 0.
    constexpr int PS = NBUF - 1;
    int i = 0, buf = 0;
    for (; i + PS <= nstrips; i += PS) {
        static_for<PS>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            strip(i + q, buf, std::integral_constant<int, q * S>{});
            buf = buf + 1 == NBUF ? 0 : buf + 1;
        });
    }
    static_for<PS - 1>([&](auto qc) __attribute__((always_inline)) {
        constexpr int q = decltype(qc)::value;
        if (i + q < nstrips) {
            strip(i + q, buf, std::integral_constant<int, q * S>{});
            buf = buf + 1 == NBUF ? 0 : buf + 1;
        }
    });
    // strip loads past the last strip still write this workgroup's LDS
    wait_vmcnt<0>();

    float* __restrict__ y = static_cast<float*>(g.y);
    const int32_t img0 = m0 / g.PQ, pq0 = m0 - img0 * g.PQ;   // image and position of the tile's first pixel
    const float rPQ = 1.0f / float(g.PQ);
    if ((g.PQ & 3) == 0) {
        // Output, bias added, straight from the accumulators: lane (gq, l16)
        // holds pixels m .. m+3 of channel n, contiguous in NKPQ (4-pixel
        // groups never straddle an image).
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int n = n0 + wn * WN + j * 16 + (lane & 15);
#pragma unroll
            for (int ii = 0; ii < TM; ++ii) {
                const int32_t rel = wm * WM + ii * 16 + 4 * (lane >> 4);
                if (n >= g.K || m0 + rel >= M) continue;
                const int32_t di = div_small(pq0 + rel, g.PQ, rPQ);
                const int32_t pq = pq0 + rel - di * g.PQ;
                store16(y + (int64_t(img0 + di) * g.K + n) * g.PQ + pq,
                        u32x4{__float_as_uint(acc[ii][j][0] + bias_v[j]), __float_as_uint(acc[ii][j][1] + bias_v[j]),
                              __float_as_uint(acc[ii][j][2] + bias_v[j]), __float_as_uint(acc[ii][j][3] + bias_v[j])});
            }
        }
        return;
    }
    // Otherwise through LDS (idle now): the tile is written channel-major,
    // bias added, then stored as runs of consecutive pixels of one channel.
    __syncthreads();
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int nl = wn * WN + j * 16 + (lane & 15);
#pragma unroll
        for (int ii = 0; ii < TM; ++ii) {
            const int ml = wm * WM + ii * 16 + 4 * (lane >> 4);
            store16(smem + nl * OP + ml,
                    u32x4{__float_as_uint(acc[ii][j][0] + bias_v[j]), __float_as_uint(acc[ii][j][1] + bias_v[j]),
                          __float_as_uint(acc[ii][j][2] + bias_v[j]), __float_as_uint(acc[ii][j][3] + bias_v[j])});
        }
    }
    __syncthreads();
    for (int t = tid; t < BN * BM; t += NT) {
        const int nl = t / BM, ml = t - (t / BM) * BM;
        const int n = n0 + nl;
        if (n >= g.K || m0 + ml >= M) continue;
        const int32_t di = div_small(pq0 + ml, g.PQ, rPQ);
        y[(int64_t(img0 + di) * g.K + n) * g.PQ + (pq0 + ml - di * g.PQ)] = smem[nl * OP + ml];
    }
}

}  // namespace convlower
