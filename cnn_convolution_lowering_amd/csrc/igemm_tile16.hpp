// 16-bit NHWC implicit contraction for small windows (few input channels,
// K <= 16*TN*SPLIT): the stem layers whose cost is writing their output.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract): every window is read from one
// copy of the input rows under its output rows.  In NHWC with unit
// horizontal dilation, the part of a window on one input row -- S pixels of
// C channels -- is one contiguous run of S*C elements of that row.  A tile
// is a block of output rows p0 .. p0+np-1 of one image; the input rows it
// touches are copied, zero-padded, into LDS once (4-byte LDS-DMA loads
// straight from x) and every pixel's window is read from there as whole
// runs.  Workgroups are persistent (a few per CU) and double-buffer the
// staging: the next tile's rows load while this tile is contracted.
//
// The contraction over one filter row is that run, preceded by `lead`
// zero-weight elements so that it starts on a 4-byte boundary, padded with
// zero weights to whole 8-element chunks (one MFMA lane group's share of a
// 32-deep step); filter row r owns chunks r*cpr .. r*cpr+cpr-1.  Only (C*sw)
// even and (W*C) even are needed for every run and every staged word to
// stay 4-byte aligned.
//
// Roles are swapped against the other contraction kernels: the filter is
// the MFMA A operand (16 output channels by 32 contraction elements, kept in
// registers for the kernel's life, loaded from a copy already in fragment
// order), the pixels are B, so each lane's accumulators hold 4*TN
// consecutive channels of one pixel.  A 16-pixel block leaves through a
// per-wave LDS buffer so that consecutive lanes store consecutive 16-byte
// pieces of the block's NHWC run.  v_mfma_f32_16x16x32_{f16,bf16}, fp32
// accumulation.
#pragma once

#include "igemm_dma.hpp"

namespace convlower {

// SPLIT waves share each block of 16 pixels, wave hc taking output
// channels hc*16*TN .. (hc+1)*16*TN - 1, so that a wave holds only its part
// of the filter and more waves fit on a SIMD.
// Persistent workgroups per CU: tile16_wgs_per_cu(tn) (register budget).
template <typename T, int KS, int TN, int SPLIT>
__global__ void __launch_bounds__(256, tile16_wgs_per_cu(TN)) conv_nhwc_tile16_kernel(GemmArgs g) {
    static_assert(TN == 2 || TN == 4, "whole 16-byte output stores");
    static_assert(SPLIT == 1 || SPLIT == 2, "four waves: 4/SPLIT pixel streams");
    constexpr int NSTREAM = 4 / SPLIT;
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ps = wave / SPLIT, hc = wave % SPLIT;   // pixel stream, channel part
    const int gq = lane >> 4, l16 = lane & 15;

    // Tiles: image n, output rows p0 .. p0+np-1 (np = tile_rows but for the
    // last block of rows), n-major.  Persistent workgroups; the tiles are cut
    // into 8 contiguous ranges, one per XCD (block b runs on XCD b % 8), and
    // the XCD's workgroups stride through its range, so that neighbouring
    // blocks of rows -- which share input rows -- meet in the same L2.
    const int P = g.PQ / g.Q;
    const int TP = g.tile_rows;
    const int tiles_p = (P + TP - 1) / TP;
    const int tiles = int(g.M / g.PQ) * tiles_p;
    const int G = int(gridDim.x), xcd = int(blockIdx.x) % 8;
    const int nw = G / 8 + (xcd < G % 8 ? 1 : 0);
    const int t_begin = xcd * (tiles / 8) + (xcd < tiles % 8 ? xcd : tiles % 8);
    const int t_end = t_begin + tiles / 8 + (xcd < tiles % 8 ? 1 : 0);
    const Tile16Geom geo = tile16_geom(g.C, g.S, g.pw);
    // Staged row: words; word u holds input elements 2(u - shift), +1 of the
    // row (zero outside it).  Long enough for the last pixel's last chunk.
    // Two staging buffers of bufw words: a tile's rows are loaded while the
    // previous tile is contracted.
    const int ldw = ((g.Q - 1) * g.sw * g.C + 8 * geo.cpr) / 2;
    const int shift = (g.pw * g.C + geo.lead) / 2;
    const int roww = g.W * g.C / 2;
    const int bufw = ((TP - 1) * g.sh + (g.R - 1) * g.dh + 1) * ldw;

    // Filter fragments (already in lane order: A[jb][st] of lane l in
    // channel part hc is 16 bytes at (((hc*TN + jb)*KS + st)*64 + l)*16) and
    // the bias, issued ahead of the
    // first staging so that all of them are in flight together.  The bias
    // loads are unconditional (a branch around each one waits for it in
    // turn): clamped channel, and without a bias the filter copy (at least
    // 1024 elements) stands in for it and its values are discarded.
    const u32x4* __restrict__ frag = static_cast<const u32x4*>(g.b);
    u32x4 af[TN][KS];
#pragma unroll
    for (int jb = 0; jb < TN; ++jb)
#pragma unroll
        for (int st = 0; st < KS; ++st) af[jb][st] = frag[((hc * TN + jb) * KS + st) * 64 + lane];
    const bool has_bias = g.bias != nullptr;
    const T* __restrict__ bsrc = static_cast<const T*>(has_bias ? g.bias : g.b);
    const int c0 = hc * 16 * TN + gq * 4 * TN;   // this lane's first output channel
    f32x4 bv[TN];                 // accumulator start: the bias of the lane's channels
#pragma unroll
    for (int jb = 0; jb < TN; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = c0 + jb * 4 + e;
            const float v = to_f32(bsrc[ch < g.K ? ch : g.K - 1]);
            bv[jb][e] = (has_bias && ch < g.K) ? v : 0.f;
        }

    const uint32_t lds0 = lds_offset(lds);
    const float rld = 1.0f / float(ldw);
    // 4-byte LDS-DMA loads of tile t's input rows h0 .. h0+rows_in-1 into
    // buffer buf, all in flight at once.
    // (t and buf are wave-uniform; readfirstlane keeps the buffer resource and
    // M0 in scalar registers, as the DMA instruction needs.)
    auto stage = [&](int tu, int bufu) __attribute__((always_inline)) {
        const int t = __builtin_amdgcn_readfirstlane(tu), buf = __builtin_amdgcn_readfirstlane(bufu);
        const int n = t / tiles_p, p0 = (t - n * tiles_p) * TP;
        const int np = P - p0 < TP ? P - p0 : TP;
        const int total = ((np - 1) * g.sh + (g.R - 1) * g.dh + 1) * ldw;
        const int h0 = p0 * g.sh - g.ph;
        const i32x4 xr = make_rsrc(static_cast<const T*>(g.a) + int64_t(n) * g.H * g.W * g.C,
                                   uint32_t(g.H * roww * 4));
        const uint32_t base = lds0 + uint32_t(buf * bufw * 4);
        for (int i0 = 0; i0 < total; i0 += 256) {
            const int i = i0 + tid;
            if (i >= total) continue;
            const int row = div_small(i, ldw, rld), u = i - row * ldw;
            const int h = h0 + row, wd = u - shift;
            const bool in = unsigned(h) < unsigned(g.H) && unsigned(wd) < unsigned(roww);
            dma4(xr, in ? uint32_t((h * roww + wd) * 4) : kOutOfRange, base + uint32_t((i0 + wave * 64) * 4));
        }
    };
    int t = t_begin + int(blockIdx.x) / 8;
    if (t < t_end) stage(t, 0);

    // Chunk st*4 + gq of the contraction: filter row r = chunk / cpr, run
    // offset 8*(chunk % cpr); past the last row the weights are zero and any
    // staged word will do.
    int off[KS];
#pragma unroll
    for (int st = 0; st < KS; ++st) {
        const int j = st * 4 + gq;
        const int r = j / geo.cpr;
        off[st] = r < g.R ? r * g.dh * ldw + (j - r * geo.cpr) * 4 : 0;
    }
    const int dp = 16 * NSTREAM / g.Q, dq = 16 * NSTREAM - (16 * NSTREAM / g.Q) * g.Q;
    const int pixw = g.sw * g.C / 2, rowstep = g.sh * ldw;
    const bool vec = (g.K & 7) == 0 && c0 + 4 * TN <= g.K;
    // Output transpose: with K = 16*TN*SPLIT each pixel of a block has a
    // run of 16*TN outputs from this wave, but each lane holds 4*TN channels
    // of one pixel, so its 16-byte stores would land 2*K bytes apart and none
    // would coalesce.  The block goes through this wave's LDS buffer instead
    // (16 pixel rows, padded by 16 bytes against bank conflicts) and leaves
    // as 16-byte pieces, consecutive lanes writing consecutive pieces.
    constexpr int XPITCH = 32 * TN + 16;
    const bool full_k = g.K == 16 * TN * SPLIT;
    char* xbuf = reinterpret_cast<char*>(lds + ((2 * bufw + 3) & ~3)) + wave * 16 * XPITCH;

    for (int it = 0; t < t_end; ++it, t += nw) {
        // Tile t's rows have landed (every wave's loads: wait, then barrier),
        // and every wave is done with the other buffer: stage the next tile.
        wait_vmcnt<0>();
        __syncthreads();
        if (t + nw < t_end) stage(t + nw, (it + 1) & 1);

        const int n = t / tiles_p, p0 = (t - n * tiles_p) * TP;
        const int np = P - p0 < TP ? P - p0 : TP;
        const uint32_t* __restrict__ sl = lds + (it & 1) * bufw;
        // Pixel blocks of 16, stream-strided: lane l16's pixel (pl, q)
        // advances by 16*NSTREAM pixels per pass without a division.
        // Software-pipelined: the next block's chunks are read, and the
        // previous block is stored, while this block's MFMAs run.
        const int count = np * g.Q;
        int ml = ps * 16 + l16;
        int pl = ml / g.Q, q = ml - (ml / g.Q) * g.Q;
        T* __restrict__ y = static_cast<T*>(g.y) + (int64_t(n) * P + p0) * g.Q * g.K;
        auto read_block = [&](u32x4 (&bq)[KS]) __attribute__((always_inline)) {
            const uint32_t* src = sl + (ml < count ? pl * rowstep + q * pixw : 0);
#pragma unroll
            for (int st = 0; st < KS; ++st) {
                const uint32_t* s = src + off[st];
                bq[st] = u32x4{s[0], s[1], s[2], s[3]};
            }
        };
        auto advance = [&]() __attribute__((always_inline)) {
            ml += 16 * NSTREAM;
            pl += dp;
            q += dq;
            if (q >= g.Q) {
                q -= g.Q;
                ++pl;
            }
        };
        // lane (gq, l16) holds channels c0 .. c0+4*TN-1 of pixel b*16 + l16
        auto store_block = [&](const f32x4 (&acc)[TN], int b) __attribute__((always_inline)) {
            if (full_k && b * 16 + 16 <= count) {
#pragma unroll
                for (int h = 0; h < TN / 2; ++h) {
                    Pack16<T> pk;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pk.e[e] = from_f32<T>(acc[2 * h + e / 4][e % 4]);
                    store16(xbuf + l16 * XPITCH + (gq * 4 * TN + 8 * h) * 2, pk.v);   // the wave's own channels
                }
                T* yb = y + int64_t(b) * 16 * g.K + hc * 16 * TN;
#pragma unroll
                for (int i = 0; i < TN / 2; ++i) {
                    const int id = lane + 64 * i;   // 16-byte piece: pixel id / (2*TN), piece id % (2*TN) of its run
                    const int px = id / (2 * TN), pc = id % (2 * TN);
                    store16(yb + px * g.K + pc * 8, load16(xbuf + px * XPITCH + pc * 16));
                }
                return;
            }
            const int m = b * 16 + l16;
            if (m >= count) return;
            T* yp = y + int64_t(m) * g.K + c0;
            if (vec) {
#pragma unroll
                for (int h = 0; h < TN / 2; ++h) {
                    Pack16<T> pk;
#pragma unroll
                    for (int e = 0; e < 8; ++e) pk.e[e] = from_f32<T>(acc[2 * h + e / 4][e % 4]);
                    store16(yp + 8 * h, pk.v);
                }
            } else {
#pragma unroll
                for (int jb = 0; jb < TN; ++jb)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (c0 + jb * 4 + e < g.K) yp[jb * 4 + e] = from_f32<T>(acc[jb][e]);
            }
        };

        u32x4 b0[KS];
        read_block(b0);
        f32x4 prev[TN];
        int b = ps;
        for (; b * 16 < count; b += NSTREAM) {
            advance();
            u32x4 b1[KS];
            read_block(b1);   // next block (a valid pixel-0 window past the end)
            f32x4 acc[TN];
#pragma unroll
            for (int jb = 0; jb < TN; ++jb) acc[jb] = bv[jb];
#pragma unroll
            for (int st = 0; st < KS; ++st)
#pragma unroll
                for (int jb = 0; jb < TN; ++jb) acc[jb] = Mfma<T>::run(af[jb][st], b0[st], acc[jb]);
            if (b != ps) store_block(prev, b - NSTREAM);
#pragma unroll
            for (int jb = 0; jb < TN; ++jb) prev[jb] = acc[jb];
#pragma unroll
            for (int st = 0; st < KS; ++st) b0[st] = b1[st];
        }
        if (b != ps) store_block(prev, b - NSTREAM);
    }
    wait_vmcnt<0>();
}

}  // namespace convlower
