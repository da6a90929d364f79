// Pipelined fused contraction for fp32 NCHW input (KCRS filter, NKPQ output).
//
// The window of an output pixel in NCHW is not a run of 16-byte chunks (its
// elements lie H*W apart), so here the A tile is stored contraction-major,
// sA[k][pixel], and filled by 4-byte LDS-DMA loads (buffer_load_dword ...
// lds): one wave-load moves one contraction element k = (c, r, s) for 64
// consecutive output pixels, i.e. 64 samples along input rows.  The element's
// tap and channel are then the same for every lane of the load, so they are
// decoded in scalar registers, and a lane's offset is its pixel's base plus a
// scalar, with two range checks for the zero padding (out-of-range lanes load
// the out-of-range offset, which writes 0).  The filter rows, contiguous in
// the same (c, r, s) order, arrive by 4-byte DMA as well, into the swizzled
// [n][k] layout of the other kernels, so any C*R*S is accepted.
//
// MFMA v_mfma_f32_16x16x4_f32: lane group g supplies contraction elements
// 4g..4g+3 of a 16-deep step, one per instruction.  A comes from four rows of
// sA (4-byte reads), B from one 16-byte chunk of its row.
//
// Sources: "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom
// PyTorch Extension", sections "Transforming Conv2D into im2col and GEMM" and
// "Global Memory and Shared Memory"; the asynchronous staging follows the
// abstract of "Enabling Memory-efficient Im2win Convolution with
// Multi-precision Support on GPU CUDA and Tensor Cores".
#pragma once

#include "igemm_dma.hpp"

namespace convlower {

// 4 bytes from rsrc+voffset into LDS at m0 + 4*lane (m0 wave-uniform); the
// builtin, as dma16.
__device__ __forceinline__ void dma4(i32x4 rsrc, uint32_t voffset, uint32_t m0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(as_rsrc(rsrc), (__attribute__((address_space(3))) void*)uintptr_t(m0), 4,
                                             voffset, 0, 0, 0);
}

// Contraction position (c, r, s) of a wave-uniform element index, stepped
// forward without division.
struct CrsCounter {
    int kk, c, r, s;
    __device__ __forceinline__ void set(int k, int R, int S) {
        kk = k;
        c = k / (R * S);
        const int rs = k - c * R * S;
        r = rs / S;
        s = rs - r * S;
    }
    __device__ __forceinline__ void step(int d, int R, int S) {
        kk += d;
        s += d;
        while (s >= S) {
            s -= S;
            if (++r == R) {
                r = 0;
                ++c;
            }
        }
    }
};

// MASK: R*S <= 32, so the valid taps of each output pixel fit in one 32-bit
// mask built once; otherwise the range checks are done per load.
template <int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool MASK>
__global__ void __launch_bounds__(256, 2) conv_nchw_f32_dma_kernel(GemmArgs g) {
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int BMP = BM + 4;                  // sA row pitch (floats), see below
    constexpr int A_ELEMS = BK * BMP;
    constexpr int B_ELEMS = BN * BK;
    constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
    constexpr int HALVES = BM / 64;               // wave-loads per A row
    constexpr int RPW = BK / 4;                   // A rows per wave per tile
    constexpr int A_LOADS = RPW * HALVES;         // per wave per tile
    constexpr int B_WLOADS = B_ELEMS / 64;        // wave-loads of the B tile
    constexpr int B_LOADS = B_WLOADS / 4;         // per wave per tile
    constexpr int BROWS = 64 / BK;                // B rows per wave-load
    constexpr int CPR = BK / 4;                   // 16-byte chunks per B row
    static_assert((BK == 16 || BK == 32) && BM % 64 == 0 && B_WLOADS % 4 == 0, "tile");
    static_assert(WGM * WGN == 4 && WM % 16 == 0 && WN % 16 == 0, "waves");
    static_assert((STAGES - 2) * (A_LOADS + B_LOADS) < 64, "vmcnt range");
    // A fragment read: lane group g reads row kb*16 + 4g + e, 16 consecutive
    // pixels; the four groups' rows are 4*BMP floats apart, 16 banks apart.
    static_assert((4 * BMP) % 64 == 16, "fragment reads on distinct banks");

    __shared__ __attribute__((aligned(16))) float smem[STAGES * STAGE_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile_m = blockIdx.x / g.tiles_n;
    const int tile_n = blockIdx.x - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;
    const int HW = g.H * g.W;

    // ---- A side.  Wave w fills A rows w*RPW .. w*RPW+RPW-1 of every tile;
    // load j covers row w*RPW + j/HALVES, pixel half h = j%HALVES (pixel
    // h*64 + lane of the tile).
    int32_t n_first, p_, q_;
    decode_m(g, int32_t(m0 < g.M ? m0 : g.M - 1), n_first, p_, q_);
    const int64_t img = int64_t(g.C) * HW;
    const int64_t n_imgs = g.M / g.PQ;
    const int64_t a_bytes = (n_imgs - n_first) * img * 4;
    const i32x4 a_rsrc = make_rsrc(static_cast<const float*>(g.a) + int64_t(n_first) * img,
                                   uint32_t(a_bytes < int64_t(0x7fffffff) ? a_bytes : int64_t(0x7fffffff)));
    int32_t pbase[HALVES];   // bytes
    int32_t ph0[HALVES], pw0[HALVES];
    uint32_t taps[HALVES];   // MASK: bit r*S+s set when tap (r, s) lies inside the image
#pragma unroll
    for (int h = 0; h < HALVES; ++h) {
        const int64_t m = m0 + h * 64 + lane;
        const bool ok = m < g.M;
        int32_t n, p, q;
        decode_m(g, ok ? int32_t(m) : 0, n, p, q);
        const int hv = p * g.sh - g.ph;
        pw0[h] = q * g.sw - g.pw;
        pbase[h] = (int32_t((n - n_first) * img) + hv * g.W + pw0[h]) * 4;
        ph0[h] = ok ? hv : -(1 << 28);   // rows past M never pass the range check
        if (MASK) {
            uint32_t t = 0;
            for (int r = 0; r < g.R; ++r)
                for (int s2 = 0; s2 < g.S; ++s2) {
                    const bool in = ok & (unsigned(hv + r * g.dh) < unsigned(g.H)) &
                                    (unsigned(pw0[h] + s2 * g.dw) < unsigned(g.W));
                    t |= uint32_t(in) << (r * g.S + s2);
                }
            taps[h] = t;
        }
    }
    CrsCounter ka;
    ka.set(wave * RPW, g.R, g.S);
    const int HW4 = HW * 4, W4 = g.W * 4;

    // ---- B side: filter rows [K][Kc] in (c, r, s) order, 4-byte loads.
    // Wave-load b covers B tile rows BROWS*b .. (BK dwords each); lane L fills
    // row BROWS*b + L/BK, LDS dword slot L%BK, which holds global element
    // 4*swz(row, slot/4) + slot%4 of that row.
    const int64_t b_last = (n0 + BN - 1 < g.K ? n0 + BN - 1 : g.K - 1);
    const i32x4 b_rsrc = make_rsrc(static_cast<const float*>(g.b) + int64_t(n0) * g.ldb,
                                   uint32_t((b_last - n0 + 1) * int64_t(g.ldb) * 4));
    int32_t bofs[B_LOADS], bcol[B_LOADS];
#pragma unroll
    for (int j = 0; j < B_LOADS; ++j) {
        const int row = BROWS * (j * 4 + wave) + lane / BK;
        const int slot = lane % BK;
        bcol[j] = 4 * swz_chunk<CPR>(row, slot / 4) + slot % 4;
        bofs[j] = (row * g.ldb + bcol[j]) * 4;                  // bytes from the tile's first row
        if (n0 + row >= g.K) bcol[j] = 1 << 28;                  // rows past K never pass
    }
    int kb0 = 0;   // contraction position of the tile being issued (B side)

    const uint32_t lds0 = lds_offset(smem);
    auto issue = [&](int st) {
        const uint32_t a_base = lds0 + uint32_t(st * STAGE_ELEMS * 4);
        const uint32_t b_base = a_base + uint32_t(A_ELEMS * 4);
#pragma unroll
        for (int j = 0; j < A_LOADS; ++j) {
            const int h = j % HALVES;
            const int kr = wave * RPW + j / HALVES;
            // ka is at contraction element k0 + kr here
            const int dh = ka.r * g.dh, dw = ka.s * g.dw;
            bool in;
            if (MASK)
                in = (ka.kk < g.Kc) & ((taps[h] >> (ka.r * g.S + ka.s)) & 1u);
            else
                in = (ka.kk < g.Kc) & (unsigned(ph0[h] + dh) < unsigned(g.H)) &
                     (unsigned(pw0[h] + dw) < unsigned(g.W));
            const int32_t o = pbase[h] + ka.c * HW4 + dh * W4 + dw * 4;
            dma4(a_rsrc, in ? uint32_t(o) : kOutOfRange, a_base + uint32_t((kr * BMP + h * 64) * 4));
            if (h == HALVES - 1) {
                if (j / HALVES == RPW - 1)
                    ka.step(BK - RPW + 1, g.R, g.S);   // to this wave's first row of the next tile
                else
                    ka.step(1, g.R, g.S);
            }
        }
#pragma unroll
        for (int j = 0; j < B_LOADS; ++j) {
            const bool in = kb0 + bcol[j] < g.Kc;
            dma4(b_rsrc, in ? uint32_t(bofs[j] + kb0 * 4) : kOutOfRange, b_base + uint32_t((j * 4 + wave) * 256));
        }
        kb0 += BK;
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = (g.Kc + BK - 1) / BK;
#pragma unroll
    for (int st = 0; st < STAGES - 1; ++st)
        if (st < nkt) issue(st);

    const int frag_row = lane & 15;
    const int grp = lane >> 4;
    for (int kt = 0; kt < nkt; ++kt) {
        if (kt + STAGES - 2 < nkt)
            wait_vmcnt<(STAGES - 2) * (A_LOADS + B_LOADS)>();
        else
            wait_vmcnt<0>();
        lds_barrier();
        const float* sA = smem + (kt % STAGES) * STAGE_ELEMS;
        const float* sB = sA + A_ELEMS;
        // Fragments of 16-deep step kb; those of step kb+1 are read while the
        // MFMAs of step kb run (sched_barrier keeps the reads ahead of them).
        f32x4 fa[2][TM], fb[2][TN];
        auto frags = [&](int kb, int buf) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const float* p = sA + (kb * 16 + 4 * grp) * BMP + wm * WM + i * 16 + frag_row;
                fa[buf][i] = f32x4{p[0], p[BMP], p[2 * BMP], p[3 * BMP]};
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 16 + frag_row;
                fb[buf][j] = __builtin_bit_cast(f32x4, load16(sB + row * BK + swz_chunk<CPR>(row, kb * 4 + grp) * 4));
            }
        };
        frags(0, 0);
#pragma unroll
        for (int kb = 0; kb < BK / 16; ++kb) {
            if (kb + 1 < BK / 16) frags(kb + 1, (kb + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[kb & 1][i][e], fb[kb & 1][j][e], acc[i][j],
                                                                         0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kt + STAGES - 1 < nkt) issue((kt + STAGES - 1) % STAGES);
    }

    // Fused epilogue through LDS: the tile is written channel-major into the
    // (now idle) pipeline buffer, bias added, then stored as 16-byte pieces
    // of contiguous NKPQ rows -- consecutive lanes write consecutive pixels
    // of one output channel, instead of 16 channels 64 bytes each.
    constexpr int OP = BM + 4;   // row pitch (floats): rows 4 banks apart for the 16-row writes
    static_assert(BN * OP <= STAGES * STAGE_ELEMS, "output tile fits the pipeline buffer");
    __syncthreads();
    {
        const float* __restrict__ bias = static_cast<const float*>(g.bias);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int nl = wn * WN + j * 16 + (lane & 15);
            const float bk = (bias && n0 + nl < g.K) ? bias[n0 + nl] : 0.f;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int ml = wm * WM + i * 16 + 4 * (lane >> 4);
                store16(smem + nl * OP + ml, u32x4{__float_as_uint(acc[i][j][0] + bk), __float_as_uint(acc[i][j][1] + bk),
                                                   __float_as_uint(acc[i][j][2] + bk), __float_as_uint(acc[i][j][3] + bk)});
            }
        }
    }
    __syncthreads();
    {
        float* __restrict__ y = static_cast<float*>(g.y);
        constexpr int G = BM / 4;                  // 4-pixel groups per channel row
        const bool vec = (g.PQ & 3) == 0;          // groups never straddle an image
        for (int t = tid; t < BN * G; t += 256) {
            const int nl = t / G, gi = t - (t / G) * G;
            const int n = n0 + nl;
            const int64_t m = m0 + 4 * gi;
            if (n >= g.K || m >= g.M) continue;
            const u32x4 v = load16(smem + nl * OP + 4 * gi);
            if (vec && m + 3 < g.M) {
                const int32_t img = int32_t(m / g.PQ);
                const int32_t pq = int32_t(m - int64_t(img) * g.PQ);
                store16(y + (int64_t(img) * g.K + n) * g.PQ + pq, v);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t me = m + e;
                    if (me >= g.M) break;
                    const int32_t img = int32_t(me / g.PQ);
                    const int32_t pq = int32_t(me - int64_t(img) * g.PQ);
                    y[(int64_t(img) * g.K + n) * g.PQ + pq] = __uint_as_float(v[e]);
                }
            }
        }
    }
}

}  // namespace convlower
