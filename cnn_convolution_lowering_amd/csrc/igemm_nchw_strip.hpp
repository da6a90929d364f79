// fp32 NCHW strip-staged implicit contraction (no horizontal padding, C a
// multiple of 16): the im2win window layout built in LDS, for the NCHW fp32
// encoder layers.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract): the window of every output pixel
// is a contiguous run of one copy of the input rows under its output row.  In
// NCHW those input rows are contiguous along w, so the copy is loaded with
// 16-byte LDS-DMA loads (four columns per lane) instead of one 4-byte gather
// per window element: for filter row r and a block of 16 input channels the
// workgroup stages rows h = p*sh - ph + r*dh (zero outside the image) of the
// output rows a tile's pixels touch, columns 0 .. W_used-1 (W_used =
// (Q-1)*sw + (S-1)*dw + 1 <= W without horizontal padding), and every tap s
// of that filter row reads its window from the same rows.  Rows are loaded
// in whole 16-byte pieces from column 0, so up to three columns past W_used
// land in the strip too (never read; past the end of x they read as zero).
//
// Contraction order: strip (cb, r) after strip, filter rows inner (so the
// rows that strips of neighbouring r share are fetched again while still in
// L2), and within a strip one 16-deep step per tap s over the block's 16
// channels; lane group
// gq = lane/16 takes channels 4*gq .. 4*gq+3 of the step, so the four
// elements of a lane lie one channel plane (a compile-time pitch) apart and
// a step's A fragment is one address add plus immediate-offset LDS reads.
// The filter is packed in that order into MFMA fragments
// (pack_filter_frag_f32_kernel) and streamed into registers DB steps ahead;
// LDS holds only a ring of NBUF strips, loaded NBUF-1 strips ahead, so the
// workgroup synchronises once per strip.  MFMA v_mfma_f32_16x16x4_f32, full
// fp32 products; memory operations are spread one per MFMA.
#pragma once

#include "igemm_nchw.hpp"
#include "igemm_strip_rb.hpp"

namespace convlower {

// The strip of one (r, 16-channel block): slot (c, t, chunk) of 16 bytes at
// (c*per_c + t*wq + chunk)*16 holds columns 4*chunk .. 4*chunk+3 of input
// row (c, t) (per_c >= rows*wq slots per channel plane); STRIP slots (a
// multiple of NT) per buffer, NL of them loaded by each lane.
template <int NT, int STRIP>
struct NchwStripSrc {
    static constexpr int NL = STRIP / NT;
    int32_t base[NL];   // bytes to x[n][c][p*sh - ph][4*chunk] for filter row 0, channel block 0
    int32_t hrow[NL];   // p*sh - ph, or far out of range for slots with no row
    i32x4 rsrc;

    // g0: first output row (n*P + p) of the tile, t_rows its rows, np the
    // output rows in all; x has fewer than 2^29 elements.
    template <int PER_C>
    __device__ __forceinline__ void init(const GemmArgs& g, int32_t g0, int32_t t_rows, int32_t np, int32_t wq,
                                         int tid) {
        const int32_t P = g.PQ / g.Q;
        const int32_t n_img = int32_t(g.M) / g.PQ;
        rsrc = make_rsrc(g.a, uint32_t(n_img * g.C * g.H * g.W * 4));
        const int32_t n0 = g0 / P, p0 = g0 - n0 * P;   // image and row of the tile's first output row
        const float rwq = 1.0f / float(wq), rP = 1.0f / float(P);
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int sl = j * NT + tid;
            const int c = sl / PER_C;
            const int rem = sl - c * PER_C;
            const int t = div_small(rem, wq, rwq);
            const int dn = div_small(p0 + t, P, rP);
            const bool ok = c < 16 && t < t_rows && g0 + t < np;
            const int32_t n = n0 + dn;
            const int32_t hv = (p0 + t - dn * P) * g.sh - g.ph;
            base[j] = ok ? ((n * g.C + c) * g.H + hv) * g.W * 4 + (rem - t * wq) * 16 : 0;
            hrow[j] = ok ? hv : -(1 << 28);
        }
    }
    // on == false: a strip past the last one (its loads write zeros)
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j, int r, int cb, bool on) const {
        const int32_t h = hrow[j] + r * g.dh;
        const int32_t o = base[j] + (cb * 16 * g.H * g.W + r * g.dh * g.W) * 4;
        return on && unsigned(h) < unsigned(g.H) ? uint32_t(o) : kOutOfRange;
    }
};

// Rows of the strip of a tile of bm pixels: a run of bm consecutive pixels
// touches at most (bm-1)/Q + 2 output rows.
__host__ __device__ inline int32_t nchw_strip_rows(int32_t bm, int64_t Q) { return int32_t((bm - 1) / Q + 2); }

template <int BM, int BN, int WGM, int WGN, int STRIP, int DB, int NBUF>
__global__ void __launch_bounds__(64 * WGM * WGN, 2) conv_nchw_f32_strip_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int NR = DB + 1;
    constexpr int BUF = STRIP * 4;   // floats per strip buffer
    using ASrc = NchwStripSrc<NT, STRIP>;
    constexpr int NLA = ASrc::NL;
    static_assert(NT == 256 && STRIP % NT == 0 && WM % 16 == 0 && WN % 16 == 0 && DB >= 1 && NBUF >= 2,
                  "tile shape");
    // Loads issued after strip j+1 when strip j ends (strip i goes out when
    // strip i-NBUF ends, after that step's filter loads): the filter loads of
    // (NBUF-1)*S - 1 steps and NBUF-2 strips, plus any output stores.  Lower
    // bounds for S >= 2 and S == 1.
    constexpr int W2 = TN * (2 * NBUF - 3) + (NBUF - 2) * NLA;
    constexpr int W1 = TN * (NBUF - 2) + (NBUF - 2) * NLA;
    static_assert(W2 < 64 && TM + TN + NLA < 64, "vmcnt range");

    constexpr int OP = BM + 4;   // pitch of the channel-major output tile in the epilogue
    constexpr int SMEM = NBUF * BUF > BN * OP ? NBUF * BUF : BN * OP;
    __shared__ __attribute__((aligned(16))) float smem[SMEM];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;

    // x has fewer than 2^29 elements here, so pixel indices fit 32 bits
    // (and every index below is non-negative and far below 2^22 where
    // div_small is used).
    const int32_t M = int32_t(g.M);
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int n0 = (tile - tile_m * g.tiles_n) * BN;
    const int32_t m0 = tile_m * BM;

    const int32_t w_used = (g.Q - 1) * g.sw + (g.S - 1) * g.dw + 1;
    const int32_t wq = (w_used + 3) / 4;               // 16-byte chunks per strip row
    const int32_t wp = 4 * wq;                         // floats per strip row
    constexpr int PER_C = nchw_strip_plane(STRIP);    // slots per channel plane
    constexpr int CH = PER_C * 4;                      // floats per channel plane
    const int32_t m_last = (m0 + BM < M ? m0 + BM : M) - 1;
    const int32_t g0 = m0 / g.Q;
    const int32_t t_rows = m_last / g.Q - g0 + 1;

    ASrc la;
    la.template init<PER_C>(g, g0, t_rows, M / g.Q, wq, tid);

    // This lane's fragment pixels: float offset (strip row, first column)
    // into a strip buffer.
    int32_t pix[TM];
    const int32_t q0 = m0 - g0 * g.Q;   // column of the tile's first pixel
    const float rQ = 1.0f / float(g.Q);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int32_t rel = wm * WM + i * 16 + (lane & 15);
        const int32_t t = div_small(q0 + rel, g.Q, rQ);
        pix[i] = m0 + rel < M ? t * wp + (q0 + rel - t * g.Q) * g.sw : 0;
    }

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

    // A fragment of a step at tap s from strip buffer buf: lane (gq, l16)
    // element e = channel 4*gq + e of the block at its pixel's window
    // column + s*dw, i.e. float offset (4*gq + e)*CH + pix + s*dw; `ro` is
    // the step's uniform part buf*BUF + s*dw.
    const int S = g.S;
    const int gq = lane >> 4;
    const float* const sl = smem + 4 * gq * CH;
    auto read_a1 = [&](u32x4& fa, int i, int ro) __attribute__((always_inline)) {
        const float* sa = sl + (pix[i] + ro);
        fa = u32x4{__float_as_uint(sa[0]), __float_as_uint(sa[CH]), __float_as_uint(sa[2 * CH]),
                   __float_as_uint(sa[3 * CH])};
    };

    const int CBN = g.C / 16;
    const int nstrips = g.R * CBN;
    const int nsteps = nstrips * S;

    // Strip stream: (nsr, ncb) is the filter row and channel block of strip
    // next_strip.
    const uint32_t lds0 = lds_offset(smem);
    int next_strip = 0, nsr = 0, ncb = 0;
    auto strip_load = [&](int buf, int j) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, nsr, ncb, next_strip < nstrips),
              lds0 + uint32_t(buf * BUF * 4) + uint32_t((j * NT + wave * 64) * 16));
    };
    auto strip_advance = [&]() __attribute__((always_inline)) {
        ++next_strip;
        if (++nsr == g.R) {
            nsr = 0;
            ++ncb;
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Prologue: strips 0 .. NBUF-1 into buffers 0 .. NBUF-1, filter
    // fragments of steps 0 .. DB-1.
#pragma unroll
    for (int sb = 0; sb < NBUF; ++sb) {
#pragma unroll
        for (int j = 0; j < NLA; ++j) strip_load(sb, j);
        strip_advance();
    }
    u32x4 fb[NR][TN];
    static_for<DB>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
        const int kp = d < nsteps ? d : 0;
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[d][j] = buffer_load16(brsrc, bfrag[j], kp * 1024);
    });
    wait_vmcnt<0>();
    lds_barrier();

    u32x4 fa0[TM], fa1[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) read_a1(fa0[i], i, 0);

    int buf_k = 0, sis = 0;   // buffer of the current strip, step (tap) within it

    // One step: MFMAs on fa0 (this step) with, one per MFMA, the A fragments
    // of step k+1 -> fa1, the filter fragments of step k+DB -> fb[RL], and on
    // the last step of a strip the loads of strip next_strip, NBUF on (into
    // the buffer of the strip that ends here, which every wave has finished
    // reading once past this step's barrier; past the last strip they write
    // zeros, so that every strip end issues the same number of loads).
    auto step = [&](int k, auto rcc) __attribute__((always_inline)) {
        constexpr int RC = decltype(rcc)::value;
        constexpr int RL = (RC + DB) % NR;
        constexpr int NM = 4 * TM * TN;
        const bool last = k + 1 == nsteps;
        const bool new_strip = !last && sis + 1 == S;
        if (new_strip) {
            // the next strip has landed for every wave, and every wave's
            // reads of this strip are done.
            if (S >= 2)
                wait_vmcnt<W2>();
            else
                wait_vmcnt<W1>();
            asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
            lds_barrier();
        }
        // buffer and tap of step k+1; past the last step the reads repeat
        // this step's
        const int buf_n = new_strip ? (buf_k + 1 == NBUF ? 0 : buf_k + 1) : buf_k;
        const int ro = buf_n * BUF + (new_strip ? 0 : last ? sis : sis + 1) * g.dw;
        const int kp = k + DB < nsteps ? k + DB : 0;
        static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
            constexpr int idx = decltype(idxc)::value;
            constexpr int e = idx / (TM * TN), i = (idx / TN) % TM, j = idx % TN;
            // (element values, not __builtin_bit_cast of the element lvalue,
            // which takes the vector's first element)
            const uint32_t av = fa0[i][e], bv = fb[RC][j][e];
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(av), __uint_as_float(bv), acc[i][j], 0, 0, 0);
            if constexpr (idx < TM) {
                read_a1(fa1[idx], idx, ro);
            } else if constexpr (idx < TM + TN) {
                fb[RL][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kp * 1024);
            } else if constexpr (idx < TM + TN + NLA) {
                if (new_strip) strip_load(buf_k, idx - TM - TN);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(TM + TN + NLA > NM ? TM + TN + NLA - NM : 0)>([&](auto rcx) __attribute__((always_inline)) {
            constexpr int idx = NM + decltype(rcx)::value;
            if constexpr (idx < TM)
                read_a1(fa1[idx], idx, ro);
            else if constexpr (idx < TM + TN)
                fb[RL][idx - TM] = buffer_load16(brsrc, bfrag[idx - TM], kp * 1024);
            else if (new_strip)
                strip_load(buf_k, idx - TM - TN);
        });
        __builtin_amdgcn_sched_barrier(0);
        if (new_strip) strip_advance();
#pragma unroll
        for (int i = 0; i < TM; ++i) fa0[i] = fa1[i];
        sis = new_strip ? 0 : sis + 1;
        buf_k = buf_n;
    };

    int k = 0;
    for (; k + NR <= nsteps; k += NR) {
        static_for<NR>([&](auto rcc) __attribute__((always_inline)) { step(k + decltype(rcc)::value, rcc); });
    }
    static_for<NR - 1>([&](auto rcc) __attribute__((always_inline)) {
        constexpr int RC = decltype(rcc)::value;
        if (k + RC < nsteps) step(k + RC, rcc);
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
            for (int i = 0; i < TM; ++i) {
                const int32_t rel = wm * WM + i * 16 + 4 * (lane >> 4);
                if (n >= g.K || m0 + rel >= M) continue;
                const int32_t di = div_small(pq0 + rel, g.PQ, rPQ);
                const int32_t pq = pq0 + rel - di * g.PQ;
                store16(y + (int64_t(img0 + di) * g.K + n) * g.PQ + pq,
                        u32x4{__float_as_uint(acc[i][j][0] + bias_v[j]), __float_as_uint(acc[i][j][1] + bias_v[j]),
                              __float_as_uint(acc[i][j][2] + bias_v[j]), __float_as_uint(acc[i][j][3] + bias_v[j])});
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
        for (int i = 0; i < TM; ++i) {
            const int ml = wm * WM + i * 16 + 4 * (lane >> 4);
            store16(smem + nl * OP + ml,
                    u32x4{__float_as_uint(acc[i][j][0] + bias_v[j]), __float_as_uint(acc[i][j][1] + bias_v[j]),
                          __float_as_uint(acc[i][j][2] + bias_v[j]), __float_as_uint(acc[i][j][3] + bias_v[j])});
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
