// Streaming 1x1 kernel (16-bit NHWC, unit stride, no padding, C = 32*KK,
// K <= 128 and a multiple of 4).
//
// With a 1x1 filter, unit stride and no padding the lowered matrix is x
// itself ("GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom
// PyTorch Extension", section "Transforming Conv2D into im2col and GEMM":
// each column of the lowered matrix is one window, here one pixel's C
// channels), so the layer is y[m][k] = b[k] + sum_c w[k][c] x[m][c] over the
// N*H*W pixel rows.  At C = K = 128 that is 128 flops per byte moved, far
// below the 16-bit MFMA ridge: the layer is a stream through HBM, and the
// kernel is built as one.  Each workgroup copies the whole filter (at most
// 32 KiB) into LDS in MFMA fragment order once, each wave takes it into
// registers from there, and then walks pixel blocks of
// 16 rows spread over the whole grid (block b, b + waves, ...), holding D
// blocks in flight in a ring of its own in LDS (LDS-DMA: each lane's 16 bytes
// land where the same lane reads them back) while it contracts and stores the
// oldest: reads and writes of different blocks overlap, instead of every tile
// loading, then computing, then storing in step with the others.
//
// Every pass issues the same loads and stores whatever the block
// (out-of-range offsets read zeros and drop stores), and the prologue issues
// the same sequence -- each block's loads followed by as many stores, out of
// range -- so the wait for a block's loads is one count known at compile
// time, the stores and the other D-1 blocks staying in flight.
#pragma once

#include "igemm_strip_rb.hpp"
#include "igemm_wide.hpp"
#include "igemm_nchw.hpp"

namespace convlower {

// KK: 32-deep contraction steps (C / 32); D: pixel blocks in flight per
// wave; MINB: workgroups per CU the register budget is set for.
template <typename T, int KK, int D, int MINB>
__global__ void __launch_bounds__(256, MINB) conv_1x1_stream_kernel(GemmArgs g) {
    constexpr int NF = 8;   // 16-channel output fragments (K <= 128)
    constexpr int E = int(sizeof(T));
    static_assert(E == 2 && KK >= 1 && KK <= 4 && D >= 1 && D * (KK + NF) < 64, "compiled shapes");
    __shared__ __attribute__((aligned(16))) T sb[NF * 16];
    __shared__ __attribute__((aligned(16))) unsigned char sf[NF * KK * 1024];
    __shared__ __attribute__((aligned(16))) unsigned char ring[4 * D * KK * 1024];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    // The filter into LDS by LDS-DMA, fragment (j, kk) at (j*KK + kk) KiB
    // (MFMA A operand: lane l holds w[j*16 + l%16][kk*32 + 8*(l/16) .. +7];
    // rows past K lie past the filter's K*C elements and read as zero), and
    // the bias beside it (zero past K, or without one; every wave writes the
    // same 256 bytes).
    const i32x4 wr = make_rsrc(g.b, uint32_t(g.K * g.C * E));
    constexpr int FCH = NF * KK * 64 / 256;   // 16-byte chunks per thread
#pragma unroll
    for (int q = 0; q < FCH; ++q) {
        const int jk = (q * 256 + wave * 64) / 64;
        const int j = jk / KK, kk = jk - (jk / KK) * KK;
        const uint32_t o = uint32_t(((j * 16 + (lane & 15)) * g.C + kk * 32 + (lane >> 4) * 8) * E);
        dma16(wr, o, lds_offset(sf) + uint32_t((q * 256 + wave * 64) * 16));
    }
    dma4(make_rsrc(g.bias, g.bias ? uint32_t(g.K * E) : 0u), uint32_t(lane * 4), lds_offset(sb));

    // Pixel fragments (MFMA B operand): lane l holds pixel l%16 of the block
    // and channels kk*32 + 8*(l/16) .. +7 of step kk -- one 16-byte load per
    // step, 64 contiguous bytes per pixel and load.  x ends at M*C elements
    // (checked below 2^31 bytes on the host); rows past M, and blocks past
    // the last, read as zero.
    const int64_t nblk = (g.M + 15) / 16;
    const int64_t gw = int64_t(blockIdx.x) * 4 + wave;
    const int64_t nw = int64_t(gridDim.x) * 4;
    const i32x4 xr = make_rsrc(g.a, uint32_t(g.M * g.C * E));
    const uint32_t lane_off = uint32_t(((lane & 15) * g.C + (lane >> 4) * 8) * E);
    // slot s of this wave's ring: step kk at kk KiB, lane l at 16*l
    const uint32_t ring_wave = lds_offset(ring) + uint32_t(wave * D * KK * 1024);
    auto issue = [&](int s, int64_t b) __attribute__((always_inline)) {
        const uint32_t o = b < nblk ? uint32_t(b * 16 * g.C * E) + lane_off : kOutOfRange;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) dma16(xr, o + uint32_t(kk * 32 * E), ring_wave + uint32_t((s * KK + kk) * 1024));
    };
    const unsigned char* ring_lane = ring + (wave * D * KK * 64 + lane) * 16;
    // Output fragments: lane l holds channels j*16 + 4*(l/16) .. +3 of
    // pixel l%16, stored as 8 bytes.  y ends at M*K elements (checked on the
    // host); a lane whose channels lie past K (K is a multiple of 4), or
    // whose pixel is past M, stores out of range.
    const int kl = 4 * (lane >> 4);
    const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(g.y, 0, int(g.M * g.K * E), 0x00020000);
    auto store_block = [&](uint32_t row_off, const f32x4* acc) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            const int k = j * 16 + kl;
            union {
                u32x2 u;
                T e[4];
            } pk, bb;
            bb.u = *reinterpret_cast<const u32x2*>(sb + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(acc[j][e] + to_f32(bb.e[e]));
            const uint32_t ov = k < g.K ? row_off + uint32_t(k * E) : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b64(pk.u, yr, int(ov), 0, 0);
        }
    };

    // Prologue: the wave's first D blocks, each followed by NF stores out of
    // range (dropped), as a pass of the loop issues them.
    static_for<D>([&](auto sc) __attribute__((always_inline)) {
        constexpr int s = decltype(sc)::value;
        issue(s, gw + s * nw);
#pragma unroll
        for (int j = 0; j < NF; ++j)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{0u, 0u}, yr, int(kOutOfRange), 0, 0);
    });

    wait_vmcnt<D * (KK + NF)>();   // the filter and bias (older than the pixel blocks)
    __syncthreads();
    u32x4 f[NF][KK];
#pragma unroll
    for (int j = 0; j < NF; ++j)
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) f[j][kk] = load16(sf + ((j * KK + kk) * 64 + lane) * 16);

    // Every wave runs the same number of blocks (the grid's largest share,
    // rounded up to the ring); blocks past the last compute on zeros and
    // store nothing.
    const int64_t per_wave = (nblk + nw - 1) / nw;
    const int64_t passes = (per_wave + D - 1) / D;
    for (int64_t it = 0; it < passes; ++it) {
        static_for<D>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            const int64_t b = gw + (it * D + s) * nw;
            // this block's loads: younger are its own stores and the loads
            // and stores of the D-1 blocks after it
            wait_vmcnt<NF + (D - 1) * (KK + NF)>();
            f32x4 acc[NF];
#pragma unroll
            for (int j = 0; j < NF; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) {
                const u32x4 bf = load16(ring_lane + (s * KK + kk) * 1024);
#pragma unroll
                for (int j = 0; j < NF; ++j) acc[j] = Mfma<T>::run(f[j][kk], bf, acc[j]);
            }
            // this slot's next block, once its reads are done
            __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
            __builtin_amdgcn_sched_barrier(0);
            issue(s, b + D * nw);
            const int64_t m = b * 16 + (lane & 15);
            store_block(b < nblk && m < g.M ? uint32_t(m * g.K * E) : kOutOfRange, acc);
        });
    }
}

}  // namespace convlower
