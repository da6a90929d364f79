// 16-bit NHWC implicit contraction for small windows (few input channels,
// K <= 16*TN): the stem layers whose cost is writing their output.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract): every window is read from one
// copy of the input rows under its output rows.  In NHWC with unit
// horizontal dilation, the part of a window on one input row -- S pixels of
// C channels -- is one contiguous run of S*C elements of that row.  A
// workgroup takes a block of output rows p0 .. p0+np-1 of one image and
// copies the input rows they touch, zero-padded, into LDS once (4-byte
// LDS-DMA loads straight from x); every pixel's window is then read from
// there as whole runs.  The contraction over one filter row is that run,
// preceded by `lead` zero-weight elements so that it starts on a 4-byte
// boundary, padded with zero weights to whole 8-element chunks (one MFMA
// lane group's share of a 32-deep step); filter row r owns chunks
// r*cpr .. r*cpr+cpr-1.  Only (C*sw) even and (W*C) even are needed for
// every run and every staged word to stay 4-byte aligned.
//
// Roles are swapped against the other contraction kernels: the filter is
// the MFMA A operand (16 output channels by 32 contraction elements, kept in
// registers for the kernel's life, loaded from a copy already in fragment
// order), the pixels are B, so each lane's accumulators hold 4*TN channels
// of one pixel (NHWC-contiguous: two 16-byte stores per pixel at TN = 4).
// v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulation.
#pragma once

#include "igemm_dma.hpp"

namespace convlower {

template <typename T, int KS, int TN>
__global__ void __launch_bounds__(256) conv_nhwc_tile16_kernel(GemmArgs g) {
    static_assert(TN == 2 || TN == 4, "whole 16-byte output stores");
    extern __shared__ __attribute__((aligned(16))) uint32_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int gq = lane >> 4, l16 = lane & 15;

    // This workgroup: image n, output rows p0 .. p0+np-1.
    const int P = g.PQ / g.Q;
    const int TP = g.tile_rows;
    const int tiles_p = (P + TP - 1) / TP;
    const int n = int(blockIdx.x) / tiles_p;
    const int p0 = (int(blockIdx.x) - n * tiles_p) * TP;
    const int np = P - p0 < TP ? P - p0 : TP;
    const int rows_in = (np - 1) * g.sh + (g.R - 1) * g.dh + 1;
    const Tile16Geom geo = tile16_geom(g.C, g.S, g.pw);
    // Staged row: words; word u holds input elements 2(u - shift), +1 of the
    // row (zero outside it).  Long enough for the last pixel's last chunk.
    const int ldw = ((g.Q - 1) * g.sw * g.C + 8 * geo.cpr) / 2;
    const int shift = (g.pw * g.C + geo.lead) / 2;
    const int roww = g.W * g.C / 2;
    const int h0 = p0 * g.sh - g.ph;
    const int total = rows_in * ldw;
    const i32x4 xr = make_rsrc(static_cast<const T*>(g.a) + int64_t(n) * g.H * g.W * g.C,
                               uint32_t(g.H * roww * 4));
    const uint32_t lds0 = lds_offset(lds);
    const float rld = 1.0f / float(ldw);
    for (int i0 = 0; i0 < total; i0 += 256) {
        const int i = i0 + tid;
        if (i >= total) continue;
        const int row = div_small(i, ldw, rld), u = i - row * ldw;
        const int h = h0 + row, wd = u - shift;
        const bool in = unsigned(h) < unsigned(g.H) && unsigned(wd) < unsigned(roww);
        dma4(xr, in ? uint32_t((h * roww + wd) * 4) : kOutOfRange, lds0 + uint32_t((i0 + wave * 64) * 4));
    }

    // Filter fragments, already in lane order: A[jb][st] of lane l is
    // 16 bytes at ((jb*KS + st)*64 + l)*16.
    const u32x4* __restrict__ frag = static_cast<const u32x4*>(g.b);
    u32x4 af[TN][KS];
#pragma unroll
    for (int jb = 0; jb < TN; ++jb)
#pragma unroll
        for (int st = 0; st < KS; ++st) af[jb][st] = frag[(jb * KS + st) * 64 + lane];
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    const int c0 = gq * 4 * TN;   // this lane's first output channel
    float bv[TN][4];
#pragma unroll
    for (int jb = 0; jb < TN; ++jb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = c0 + jb * 4 + e;
            bv[jb][e] = (bias && ch < g.K) ? to_f32(bias[ch]) : 0.f;
        }
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
    wait_vmcnt<0>();
    __syncthreads();

    // Pixel blocks of 16, wave-strided: lane l16's pixel (pl, q) advances by
    // 64 pixels per pass without a division.  Software-pipelined as the
    // fp32 small-window kernel: the next block's chunks are read, and the
    // previous block is stored, while this block's MFMAs run.
    const int count = np * g.Q;
    const int dp = 64 / g.Q, dq = 64 - (64 / g.Q) * g.Q;
    const int pixw = g.sw * g.C / 2, rowstep = g.sh * ldw;
    int ml = wave * 16 + l16;
    int pl = ml / g.Q, q = ml - (ml / g.Q) * g.Q;
    T* __restrict__ y = static_cast<T*>(g.y) + (int64_t(n) * P + p0) * g.Q * g.K;
    const bool vec = (g.K & 7) == 0 && c0 + 4 * TN <= g.K;
    auto read_block = [&](u32x4 (&bq)[KS]) __attribute__((always_inline)) {
        const uint32_t* src = lds + (ml < count ? pl * rowstep + q * pixw : 0);
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const uint32_t* s = src + off[st];
            bq[st] = u32x4{s[0], s[1], s[2], s[3]};
        }
    };
    auto advance = [&]() __attribute__((always_inline)) {
        ml += 64;
        pl += dp;
        q += dq;
        if (q >= g.Q) {
            q -= g.Q;
            ++pl;
        }
    };
    // lane (gq, l16) holds channels c0 .. c0+4*TN-1 of pixel b*16 + l16
    auto store_block = [&](const f32x4 (&acc)[TN], int b) __attribute__((always_inline)) {
        const int m = b * 16 + l16;
        if (m >= count) return;
        T* yp = y + int64_t(m) * g.K + c0;
        if (vec) {
#pragma unroll
            for (int h = 0; h < TN / 2; ++h) {
                Pack16<T> pk;
#pragma unroll
                for (int e = 0; e < 8; ++e) pk.e[e] = from_f32<T>(acc[2 * h + e / 4][e % 4] + bv[2 * h + e / 4][e % 4]);
                store16(yp + 8 * h, pk.v);
            }
        } else {
#pragma unroll
            for (int jb = 0; jb < TN; ++jb)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (c0 + jb * 4 + e < g.K) yp[jb * 4 + e] = from_f32<T>(acc[jb][e] + bv[jb][e]);
        }
    };

    u32x4 b0[KS];
    read_block(b0);
    f32x4 prev[TN];
    int b = wave;
    for (; b * 16 < count; b += 4) {
        advance();
        u32x4 b1[KS];
        read_block(b1);   // next block (a valid pixel-0 window past the end)
        f32x4 acc[TN];
#pragma unroll
        for (int jb = 0; jb < TN; ++jb) acc[jb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int jb = 0; jb < TN; ++jb) acc[jb] = Mfma<T>::run(af[jb][st], b0[st], acc[jb]);
        if (b != wave) store_block(prev, b - 4);
#pragma unroll
        for (int jb = 0; jb < TN; ++jb) prev[jb] = acc[jb];
#pragma unroll
        for (int st = 0; st < KS; ++st) b0[st] = b1[st];
    }
    if (b != wave) store_block(prev, b - 4);
}

}  // namespace convlower
