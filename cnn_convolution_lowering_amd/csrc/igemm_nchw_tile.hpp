// fp32 NCHW implicit contraction for small windows (C*R*S <= 16*KS, K <=
// 16*TN): the encoder's first layer, whose cost is writing its output.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract): every window is read from one
// copy of the input rows under its output rows.  A workgroup takes a block
// of output rows p0 .. p0+np-1 of one image, copies the input rows they
// touch, zero-padded, into LDS once (one plane of rows_in x PWd floats per
// channel, PWd = (Q-1)*sw + (S-1)*dw + 1 padded columns, plus one plane of
// zeros that the padded contraction elements past C*R*S read), and reads
// every pixel's window from there.  The whole filter lives in registers as MFMA
// A fragments for the kernel's life (loaded from KCRS directly: no packed
// copy), the pixels are the B operand, so the loop is LDS reads,
// v_mfma_f32_16x16x4_f32 (full fp32 products) and 4-byte stores in which
// 16 consecutive lanes write 16 consecutive pixels of one output channel
// (one 64-byte run per lane group: the stores coalesce).  Contraction order
// k = (c*R + r)*S + s, the filter's own.
#pragma once

#include "igemm_dma.hpp"
#include "igemm_nchw.hpp"

namespace convlower {

template <int KS, int TN>
__global__ void __launch_bounds__(256) conv_nchw_f32_tile_kernel(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
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
    const int PWd = (g.Q - 1) * g.sw + (g.S - 1) * g.dw + 1;
    const int plane = rows_in * PWd;

    // Stage, with 4-byte LDS-DMA loads (all in flight at once): the input
    // rows h0 .. h0+rows_in-1, columns -pw .. PWd-pw-1 of every channel,
    // zero outside the image; the zero plane; the filter as a zero-padded
    // [16*TN][16*KS] block (KCRS rows are contiguous in k = (c*R + r)*S + s);
    // and the bias, zero-padded to 16*TN channels (zero without one).
    const int h0 = p0 * g.sh - g.ph;
    const int staged = g.C * plane;
    const int RS = g.R * g.S, Kg = g.C * RS;
    constexpr int KP = 16 * KS;
    const int fil0 = (staged + plane + 3) & ~3;   // 16-byte aligned for the fragment reads
    const int bias0 = fil0 + 16 * TN * KP;
    const int total = bias0 + 16 * TN;
    const i32x4 xr = make_rsrc(static_cast<const float*>(g.a) + int64_t(n) * g.C * g.H * g.W,
                               uint32_t(g.C * g.H * g.W * 4));
    const i32x4 wr = make_rsrc(g.b, uint32_t(g.K * Kg * 4));
    const i32x4 br = make_rsrc(g.bias ? g.bias : g.b, g.bias ? uint32_t(g.K * 4) : 0u);
    const uint32_t lds0 = lds_offset(lds);
    const float rPWd = 1.0f / float(PWd), rrows = 1.0f / float(rows_in);
    for (int i0 = 0; i0 < total; i0 += 256) {
        const int i = i0 + tid;
        if (i >= total) continue;
        const uint32_t m0 = lds0 + uint32_t((i0 + wave * 64) * 4);
        if (i < fil0) {   // input rows, the zero plane and up to 3 pad floats (zero)
            const int row = div_small(i, PWd, rPWd), j = i - row * PWd;
            const int c = div_small(row, rows_in, rrows), h = h0 + (row - c * rows_in), w = j - g.pw;
            const bool in = i < staged && unsigned(h) < unsigned(g.H) && unsigned(w) < unsigned(g.W);
            dma4(xr, in ? uint32_t(((c * g.H + h) * g.W + w) * 4) : kOutOfRange, m0);
        } else if (i < bias0) {
            const int f = i - fil0, ch = f / KP, k = f - (f / KP) * KP;
            dma4(wr, (ch < g.K && k < Kg) ? uint32_t((ch * Kg + k) * 4) : kOutOfRange, m0);
        } else {
            dma4(br, uint32_t((i - bias0) * 4), m0);   // past K (or no bias): out of range, zero
        }
    }

    // Per-lane contraction elements: step st, element e is k = st*16 +
    // 4*gq + e at LDS offset c*plane + r*dh*PWd + s*dw from the pixel's
    // window origin (the zero plane for k >= C*R*S).
    int off[KS][4];
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = st * 16 + 4 * gq + e;
            const int c = k / RS, rs = k - (k / RS) * RS;
            const int r = rs / g.S, s = rs - (rs / g.S) * g.S;
            off[st][e] = k < Kg ? c * plane + r * g.dh * PWd + s * g.dw : staged;
        }
    wait_vmcnt<0>();
    __syncthreads();
    // Bias of the lane's output channels jb*16 + 4*gq + e: the accumulators'
    // start.
    f32x4 bv[TN];
#pragma unroll
    for (int jb = 0; jb < TN; ++jb) bv[jb] = __builtin_bit_cast(f32x4, load16(lds + bias0 + jb * 16 + 4 * gq));
    // Filter fragments: lane (gq, l16) of block jb, step st holds
    // w[jb*16 + l16][st*16 + 4*gq + e] (row l16 of the A operand).
    float bf[TN][KS][4];
#pragma unroll
    for (int jb = 0; jb < TN; ++jb)
#pragma unroll
        for (int st = 0; st < KS; ++st) {
            const f32x4 v = __builtin_bit_cast(f32x4, load16(lds + fil0 + (jb * 16 + l16) * KP + st * 16 + 4 * gq));
#pragma unroll
            for (int e = 0; e < 4; ++e) bf[jb][st][e] = v[e];
        }

    // Pixel blocks of 16, wave-strided: lane l16's pixel (pl, q) advances
    // by 64 pixels per pass without a division.  Software-pipelined: the
    // window values of the next block are read, and the previous block is
    // stored, while this block's MFMAs run.
    const int count = np * g.Q;
    const int dp = 64 / g.Q, dq = 64 - (64 / g.Q) * g.Q;
    int ml = wave * 16 + l16;
    int pl = ml / g.Q, q = ml - (ml / g.Q) * g.Q;
    float* __restrict__ y = static_cast<float*>(g.y) + int64_t(n) * g.K * g.PQ + p0 * g.Q;
    auto read_block = [&](float (&a)[KS][4]) __attribute__((always_inline)) {
        const float* src = lds + (ml < count ? pl * g.sh * PWd + q * g.sw : 0);
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) a[st][e] = src[off[st][e]];
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
    // lane (gq, l16) holds channels jb*16 + 4*gq + e of pixel b*16 + l16
    auto store_block = [&](const f32x4 (&acc)[TN], int b) __attribute__((always_inline)) {
        const int m = b * 16 + l16;
        if (m >= count) return;
#pragma unroll
        for (int jb = 0; jb < TN; ++jb)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ch = jb * 16 + 4 * gq + e;
                if (ch < g.K) y[int64_t(ch) * g.PQ + m] = acc[jb][e];
            }
    };

    float a0[KS][4];
    read_block(a0);
    f32x4 prev[TN];
    int b = wave;
    for (; b * 16 < count; b += 4) {
        advance();
        float a1[KS][4];
        read_block(a1);   // next block (a valid pixel-0 window past the end)
        f32x4 acc[TN];
#pragma unroll
        for (int jb = 0; jb < TN; ++jb) acc[jb] = bv[jb];
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int jb = 0; jb < TN; ++jb)
                    acc[jb] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[jb][st][e], a0[st][e], acc[jb], 0, 0, 0);
        if (b != wave) store_block(prev, b - 4);
#pragma unroll
        for (int jb = 0; jb < TN; ++jb) prev[jb] = acc[jb];
#pragma unroll
        for (int st = 0; st < KS; ++st)
#pragma unroll
            for (int e = 0; e < 4; ++e) a0[st][e] = a1[st][e];
    }
    if (b != wave) store_block(prev, b - 4);
}

}  // namespace convlower
