// Contraction launchers: pick the kernel, tile variant and operand loaders
// recorded in the descriptor and enqueue the contraction with its fused
// epilogue.  Included once per storage type (contract_f32.hip,
// contract_f16.hip, contract_bf16.hip) so the kernels of the three types
// compile in parallel.
#pragma once

#include "dispatch.hpp"
#include "igemm.hpp"
#include "igemm_dma.hpp"
#include "igemm_nchw.hpp"
#include "igemm_nchw_strip.hpp"
#include "igemm_nchw_taps.hpp"
#include "igemm_nchw_tile.hpp"
#include "igemm_strip.hpp"
#include "igemm_strip_rb.hpp"
#include "igemm_strip_rb2.hpp"
#include "igemm_strip_rb3.hpp"
#include "igemm_strip_rb4.hpp"
#include "igemm_stream1x1.hpp"
#include "igemm_streamk.hpp"
#include "igemm_tile16.hpp"
#include "igemm_wide.hpp"

static_assert(int(convlower::TILE_ORDER_LINEAR) == int(CONV_TILE_LINEAR) &&
                  int(convlower::TILE_ORDER_XCD_ROWS) == int(CONV_TILE_XCD_ROWS) &&
                  int(convlower::TILE_ORDER_XCD_SERPENT) == int(CONV_TILE_XCD_SERPENT) &&
                  int(convlower::TILE_ORDER_XCD_COLS) == int(CONV_TILE_XCD_COLS),
              "tile order numbering");

namespace convlower {

template <typename T, int BM, int BN, int BK, int WGM, int WGN, bool NHWC_OUT, class ALoad, class BLoad>
void launch_core(const conv_desc& d, GemmArgs g, hipStream_t st) {
    g.tiles_n = int32_t((d.p.K + BN - 1) / BN);
    const uint64_t tiles_m = (uint64_t(d.M) + BM - 1) / BM;
    const uint32_t blocks = uint32_t(tiles_m * g.tiles_n);
    conv_gemm_kernel<T, BM, BN, BK, WGM, WGN, NHWC_OUT, ALoad, BLoad><<<blocks, 256, 0, st>>>(g);
}

// Pick the loaders for the descriptor and launch one tile shape.
template <typename T, int BM, int BN, int BK, int WGM, int WGN>
void launch_gemm_tile(const conv_desc& d, const GemmArgs& g, hipStream_t st) {
    constexpr int VEC = Vec<T>::n;
    using BRows = StridedRows<T, BN, BK, false, false>;
    using BRowsElem = StridedRows<T, BN, BK, false, true>;
    const bool nhwc = d.p.layout == CONV_NHWC;
    if (d.p.algo != CONV_ALGO_IMPLICIT) {
        // lowered buffer (im2win strips / im2col rows) or 1x1 NHWC input in place
        const bool seg = !d.elided && d.p.algo == CONV_ALGO_IM2WIN;
        if constexpr (sizeof(T) == 4) {
            if (d.unpadded) {
                // unpadded fp32 rows and packed filter rows: element gathers
                if (seg) {
                    using A = StridedRows<T, BM, BK, true, true>;
                    if (nhwc) launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRowsElem>(d, g, st);
                    else launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRowsElem>(d, g, st);
                } else {
                    using A = StridedRows<T, BM, BK, false, true>;
                    if (nhwc) launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRowsElem>(d, g, st);
                    else launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRowsElem>(d, g, st);
                }
                return;
            }
        }
        if (seg) {
            using A = StridedRows<T, BM, BK, true, false>;
            if (nhwc) launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRows>(d, g, st);
            else launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRows>(d, g, st);
        } else {
            using A = StridedRows<T, BM, BK, false, false>;
            if (nhwc) launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRows>(d, g, st);
            else launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRows>(d, g, st);
        }
        return;
    }
    const bool b_vec = d.Kg % VEC == 0;
    if (nhwc && d.p.C % VEC == 0) {
        launch_core<T, BM, BN, BK, WGM, WGN, true, WindowVecNHWC<T, BM, BK>, BRows>(d, g, st);
    } else if (nhwc) {
        using A = WindowElem<T, BM, BK, true>;
        if (b_vec) launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRows>(d, g, st);
        else launch_core<T, BM, BN, BK, WGM, WGN, true, A, BRowsElem>(d, g, st);
    } else {
        using A = WindowElem<T, BM, BK, false>;
        if (b_vec) launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRows>(d, g, st);
        else launch_core<T, BM, BN, BK, WGM, WGN, false, A, BRowsElem>(d, g, st);
    }
}

template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool WIDE, bool NHWC_OUT, class ASrc,
          class BSrc, int EPI = 0, bool EARLY = false>
void launch_dma_core(const conv_desc& d, GemmArgs g, hipStream_t st) {
    g.tiles_n = int32_t((d.p.K + BN - 1) / BN);
    const uint64_t tiles_m = (uint64_t(d.M) + BM - 1) / BM;
    const dim3 blocks(uint32_t(tiles_m * g.tiles_n), uint32_t(EPI || g.ksplit < 1 ? 1 : g.ksplit));
    constexpr int NT = 64 * WGM * WGN;
    if constexpr (WIDE)
        conv_gemm_wide_kernel<T, BM, BN, BK, WGM, WGN, STAGES, ASrc, BSrc><<<blocks, NT, 0, st>>>(g);
    else
        conv_gemm_dma_kernel<T, BM, BN, BK, WGM, WGN, STAGES, NHWC_OUT, ASrc, BSrc, EPI, EARLY><<<blocks, NT, 0, st>>>(g);
}

template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int BST>
void launch_strip(const conv_desc& d, GemmArgs g, hipStream_t st) {
    g.tiles_n = int32_t((d.p.K + BN - 1) / BN);
    const uint64_t tiles_m = (uint64_t(d.M) + BM - 1) / BM;
    const uint32_t blocks = uint32_t(tiles_m * g.tiles_n);
    conv_strip_kernel<T, BM, BN, WGM, WGN, STRIP, BST><<<blocks, 64 * WGM * WGN, 0, st>>>(g);
}

// Pick the DMA sources for the descriptor and launch one tile shape of the
// pipelined kernel (WIDE: the one-wave-per-SIMD schedule, implicit NHWC
// windows with C a multiple of BK only -- checked when planning).
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool WIDE, bool EARLY = false>
void launch_dma_tile(const conv_desc& d, const GemmArgs& g, hipStream_t st) {
    constexpr int NT = 64 * WGM * WGN;
    using B = DmaRows<T, BN, BK, false, false, NT>;
    const bool nhwc = d.p.layout == CONV_NHWC;
    if constexpr (WIDE) {
        using BW = DmaRows<T, BN, BK, false, false, NT, 1>;
        launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, true, true, DmaWindowNHWCBlocked<T, BM, BK, NT, 1>, BW>(d, g,
                                                                                                              st);
    } else if (d.p.algo == CONV_ALGO_IMPLICIT) {
        // NHWC with C a whole number of vectors (checked when planning)
        if (d.p.C % BK == 0)
            launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, true, DmaWindowNHWCBlocked<T, BM, BK, NT>, B, 0, EARLY>(
                d, g, st);
        else
            launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, true, DmaWindowNHWC<T, BM, BK, NT>, B, 0, EARLY>(d, g, st);
    } else if (!d.elided && d.p.algo == CONV_ALGO_IM2WIN) {
        using A = DmaRows<T, BM, BK, true, true, NT>;
        if (nhwc) launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, true, A, B, 0, EARLY>(d, g, st);
        else launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, false, A, B, 0, EARLY>(d, g, st);
    } else {
        using A = DmaRows<T, BM, BK, true, false, NT>;
        if (nhwc) launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, true, A, B, 0, EARLY>(d, g, st);
        else launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, false, A, B, 0, EARLY>(d, g, st);
    }
}

// The stream-K form of one pipelined tile shape (its operand sources as in
// launch_dma_tile): sk_grid persistent workgroups; sum slots and flags in the
// workspace's partial area.
template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES>
void launch_streamk_tile(const conv_desc& d, GemmArgs g, uint32_t epoch, hipStream_t st) {
    constexpr int NT = 64 * WGM * WGN;
    using B = DmaRows<T, BN, BK, false, false, NT>;
    g.tiles_n = int32_t((d.p.K + BN - 1) / BN);
    StreamKArgs sk;
    sk.part = static_cast<float*>(g.part);
    sk.flags = reinterpret_cast<uint32_t*>(sk.part + int64_t(d.sk_grid) * BM * BN);
    sk.epoch = epoch;
    sk.tiles = int32_t(((d.M + BM - 1) / BM) * g.tiles_n);
    sk.nkt = int32_t((g.Kc + BK - 1) / BK);
    sk.grid = d.sk_grid;
    const bool nhwc = d.p.layout == CONV_NHWC;
    const dim3 grid(uint32_t(d.sk_grid));
    if (d.p.algo == CONV_ALGO_IMPLICIT) {
        // NHWC windows of whole BK-channel blocks (checked when planning)
        conv_gemm_streamk_kernel<T, BM, BN, BK, WGM, WGN, STAGES, true, DmaWindowNHWCBlocked<T, BM, BK, NT>, B>
            <<<grid, NT, 0, st>>>(g, sk);
    } else if (!d.elided && d.p.algo == CONV_ALGO_IM2WIN) {
        using A = DmaRows<T, BM, BK, true, true, NT>;
        if (nhwc) conv_gemm_streamk_kernel<T, BM, BN, BK, WGM, WGN, STAGES, true, A, B><<<grid, NT, 0, st>>>(g, sk);
        else conv_gemm_streamk_kernel<T, BM, BN, BK, WGM, WGN, STAGES, false, A, B><<<grid, NT, 0, st>>>(g, sk);
    } else {
        using A = DmaRows<T, BM, BK, true, false, NT>;
        if (nhwc) conv_gemm_streamk_kernel<T, BM, BN, BK, WGM, WGN, STAGES, true, A, B><<<grid, NT, 0, st>>>(g, sk);
        else conv_gemm_streamk_kernel<T, BM, BN, BK, WGM, WGN, STAGES, false, A, B><<<grid, NT, 0, st>>>(g, sk);
    }
}

// The split contraction's reduction (after the contraction on the same
// stream); nothing without a split.
template <typename T>
void launch_split_reduce(const conv_desc& d, const GemmArgs& g, const void* bias, void* y, hipStream_t st) {
    if (d.ksplit <= 1) return;
    SplitReduceArgs a{static_cast<const float*>(g.part), bias, y, d.M * d.p.K, int32_t(d.p.K),
                      int32_t(d.P * d.Q), d.ksplit, d.p.layout == CONV_NHWC ? 1 : 0};
    const uint64_t work = (uint64_t(a.total) + 1023) / 1024;
    const uint32_t rblocks = uint32_t(work < 256 * 16 ? (work ? work : 1) : 256 * 16);
    splitk_reduce_kernel<T><<<rblocks, 256, 0, st>>>(a);
}

template <typename T>
void launch_gemm(const conv_desc& d, const void* x, const void* w, const void* bias, void* y, const void* ws,
                 uint32_t epoch, hipStream_t st) {
    const char* wsb = static_cast<const char*>(ws);
    GemmArgs g{};
    g.ksplit = d.ksplit;
    g.tile_order = d.tile_order;
    g.part = d.bytes_part ? static_cast<void*>(const_cast<char*>(wsb) + d.off_part) : nullptr;
    g.b = (d.pack || d.frag_pack) ? static_cast<const void*>(wsb + d.off_filter) : w;
    g.bias = bias;
    g.y = y;
    g.M = d.M;
    g.K = int32_t(d.p.K);
    g.PQ = int32_t(d.P * d.Q);
    g.Q = int32_t(d.Q);
    g.C = int32_t(d.p.C);
    g.H = int32_t(d.p.H);
    g.W = int32_t(d.p.W);
    g.R = int32_t(d.p.R);
    g.S = int32_t(d.p.S);
    g.sh = d.p.stride_h;
    g.sw = d.p.stride_w;
    g.ph = d.p.pad_h;
    g.pw = d.p.pad_w;
    g.dh = d.p.dil_h;
    g.dw = d.p.dil_w;
    if (d.p.algo == CONV_ALGO_IMPLICIT) {
        // windows gathered from x; filter rows in their own order
        g.a = x;
        g.Kc = int32_t(d.Kg);
        g.ldb = int32_t(d.Kg);
    } else if (d.elided) {
        // 1x1, no padding, NHWC: row (n, p, q) is x[n][p*sh][q*sw][0..C)
        g.a = x;
        g.Kc = int32_t(d.Kl);
        g.ldb = int32_t(d.Kl);
        g.sN = d.p.H * d.p.W * d.p.C;
        g.sP = int64_t(d.p.stride_h) * d.p.W * d.p.C;
        g.sQ = int64_t(d.p.stride_w) * d.p.C;
        g.RCp = int32_t(d.Kl);
        g.sS = 0;
    } else if (d.p.algo == CONV_ALGO_IM2WIN) {
        g.a = wsb + d.off_low;
        g.Kc = int32_t(d.Kl);
        g.ldb = int32_t(d.Kl);
        g.sP = d.W_used * d.RCp;
        g.sN = d.P * g.sP;
        g.sQ = int64_t(d.p.stride_w) * d.RCp;
        g.RCp = int32_t(d.RCp);
        g.sS = int32_t(int64_t(d.p.dil_w) * d.RCp);
    } else {
        g.a = wsb + d.off_low;
        g.Kc = int32_t(d.Kl);
        g.ldb = int32_t(d.Kl);
        g.sQ = d.Kl;
        g.sP = d.Q * d.Kl;
        g.sN = d.P * g.sP;
        g.RCp = int32_t(d.Kl);
        g.sS = 0;
    }
    if (d.kernel == KERN_NCHW) {
        if constexpr (sizeof(T) == 4) {
            auto launch = [&](auto kernel, int BM, int BN) {
                GemmArgs h = g;
                h.tiles_n = int32_t((d.p.K + BN - 1) / BN);
                const uint32_t blocks = uint32_t(((uint64_t(d.M) + BM - 1) / BM) * h.tiles_n);
                kernel<<<blocks, 256, 0, st>>>(h);
            };
            const bool mask = d.p.R * d.p.S <= 32;
#define CONVLOWER_NCHW_CASE(I)                                                                                 \
    case I: {                                                                                                  \
        constexpr TileVariant v = kNchwVariants[I];                                                            \
        if (mask) launch(conv_nchw_f32_dma_kernel<v.bm, v.bn, v.bk, v.wgm, v.wgn, v.stages, true>, v.bm, v.bn); \
        else launch(conv_nchw_f32_dma_kernel<v.bm, v.bn, v.bk, v.wgm, v.wgn, v.stages, false>, v.bm, v.bn);    \
        break;                                                                                                 \
    }
            switch (d.variant) {
                CONVLOWER_NCHW_CASE(0)
                CONVLOWER_NCHW_CASE(1)
                CONVLOWER_NCHW_CASE(2)
                CONVLOWER_NCHW_CASE(3)
                CONVLOWER_NCHW_CASE(4)
                CONVLOWER_NCHW_CASE(5)
                CONVLOWER_NCHW_CASE(6)
                CONVLOWER_NCHW_CASE(7)
                CONVLOWER_NCHW_CASE(8)
                CONVLOWER_NCHW_CASE(9)
                CONVLOWER_NCHW_CASE(10)
                CONVLOWER_NCHW_CASE(11)
                default: break;
            }
#undef CONVLOWER_NCHW_CASE
        }
        return;
    }
    // BK of a variant is given for 16-bit storage; fp32 rows of the same bytes hold half as many elements.
    constexpr int DIV = sizeof(T) == 4 ? 2 : 1;
    if (d.kernel == KERN_STREAMK) {
#define CONVLOWER_SK_CASE(I)                                                                        \
    case I: {                                                                                       \
        constexpr TileVariant v = kDmaVariants[I];                                                  \
        launch_streamk_tile<T, v.bm, v.bn, v.bk / DIV, v.wgm, v.wgn, v.stages>(d, g, epoch, st);   \
        break;                                                                                      \
    }
        switch (d.variant) {
            CONVLOWER_SK_CASE(8)
            default: break;
        }
#undef CONVLOWER_SK_CASE
        return;
    }
    if (d.kernel == KERN_DMA) {
#define CONVLOWER_DMA_CASE(I)                                                                     \
    case I: {                                                                                     \
        constexpr TileVariant v = kDmaVariants[I];                                                \
        launch_dma_tile<T, v.bm, v.bn, v.bk / DIV, v.wgm, v.wgn, v.stages, false, v.early != 0>(d, g, st); \
        break;                                                                                    \
    }
        switch (d.variant) {
            CONVLOWER_DMA_CASE(0)
            CONVLOWER_DMA_CASE(1)
            CONVLOWER_DMA_CASE(2)
            CONVLOWER_DMA_CASE(3)
            CONVLOWER_DMA_CASE(4)
            CONVLOWER_DMA_CASE(5)
            CONVLOWER_DMA_CASE(6)
            CONVLOWER_DMA_CASE(7)
            CONVLOWER_DMA_CASE(8)
            CONVLOWER_DMA_CASE(9)
            CONVLOWER_DMA_CASE(10)
            CONVLOWER_DMA_CASE(11)
            CONVLOWER_DMA_CASE(12)
            CONVLOWER_DMA_CASE(13)
            default: break;
        }
#undef CONVLOWER_DMA_CASE
        launch_split_reduce<T>(d, g, bias, y, st);
        return;
    }
    if (d.kernel == KERN_NCHW_TILE) {
        if constexpr (sizeof(T) == 4) {
            GemmArgs h = g;
            h.tile_rows = d.tile_rows;
            const int64_t P = d.P, TP = d.tile_rows;
            const uint32_t blocks = uint32_t(d.p.N * ((P + TP - 1) / TP));
            const int64_t rows_in = (TP - 1) * d.p.stride_h + (d.p.R - 1) * d.p.dil_h + 1;
            // C planes, a zero plane, the padded filter and the padded bias
            const int64_t tn = kNchwTileVariants[d.variant].tn, ks = kNchwTileVariants[d.variant].ks;
            const size_t lds = size_t(((d.p.C + 1) * rows_in * d.W_used + 3 + 256 * tn * ks + 16 * tn) * 4);
#define CONVLOWER_NCHW_TILE_CASE(I)                                                                            \
    case I:                                                                                                    \
        conv_nchw_f32_tile_kernel<kNchwTileVariants[I].ks, kNchwTileVariants[I].tn><<<blocks, 256, lds, st>>>(h); \
        break;
            switch (d.variant) {
                CONVLOWER_NCHW_TILE_CASE(0)
                CONVLOWER_NCHW_TILE_CASE(1)
                CONVLOWER_NCHW_TILE_CASE(2)
                CONVLOWER_NCHW_TILE_CASE(3)
                CONVLOWER_NCHW_TILE_CASE(4)
                CONVLOWER_NCHW_TILE_CASE(5)
                default: break;
            }
#undef CONVLOWER_NCHW_TILE_CASE
        }
        return;
    }
    if (d.kernel == KERN_TILE16) {
        if constexpr (sizeof(T) == 2) {
            GemmArgs h = g;
            h.tile_rows = d.tile_rows;
            const int64_t P = d.P, TP = d.tile_rows;
            const int64_t tiles = d.p.N * ((P + TP - 1) / TP);
            const int64_t wgs = kTile16Cus * tile16_wgs_per_cu(kTile16Variants[d.variant].tn);
            const uint32_t blocks = uint32_t(tiles < wgs ? tiles : wgs);
            const int64_t rows_in = (TP - 1) * d.p.stride_h + (d.p.R - 1) * d.p.dil_h + 1;
            const Tile16Geom geo = tile16_geom(int(d.p.C), int(d.p.S), int(d.p.pad_w));
            // two staging buffers (rounded to 16 bytes), then four waves' output
            // transpose buffers of 16 rows of 32*tn + 16 bytes
            const int64_t bufw = rows_in * ((d.Q - 1) * d.p.stride_w * d.p.C + 8 * geo.cpr) / 2;
            const size_t lds = size_t(((2 * bufw + 3) & ~int64_t(3)) * 4 +
                                      64 * (32 * kTile16Variants[d.variant].tn + 16));
#define CONVLOWER_TILE16_CASE(I)                                                                          \
    case I: {                                                                                             \
        constexpr Tile16Variant v = kTile16Variants[I];                                                   \
        conv_nhwc_tile16_kernel<T, v.ks, v.tn, v.split><<<blocks, 256, lds, st>>>(h);                     \
        break;                                                                                            \
    }
            switch (d.variant) {
                CONVLOWER_TILE16_CASE(0)
                CONVLOWER_TILE16_CASE(1)
                CONVLOWER_TILE16_CASE(2)
                CONVLOWER_TILE16_CASE(3)
                CONVLOWER_TILE16_CASE(4)
                CONVLOWER_TILE16_CASE(5)
                CONVLOWER_TILE16_CASE(6)
                CONVLOWER_TILE16_CASE(7)
                CONVLOWER_TILE16_CASE(8)
                CONVLOWER_TILE16_CASE(9)
                CONVLOWER_TILE16_CASE(10)
                default: break;
            }
#undef CONVLOWER_TILE16_CASE
        }
        return;
    }
    if (d.kernel == KERN_NCHW_STRIP) {
        if constexpr (sizeof(T) == 4) {
#define CONVLOWER_NCHW_STRIP_CASE(I)                                                                          \
    case I: {                                                                                                 \
        constexpr NchwStripVariant v = kNchwStripVariants[I];                                                 \
        GemmArgs h = g;                                                                                       \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                       \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                   \
        conv_nchw_f32_strip_kernel<v.bm, v.bn, v.wgm, v.wgn, v.strip, v.db, v.nbuf><<<blocks, 256, 0, st>>>(h); \
        break;                                                                                                \
    }
            switch (d.variant) {
                CONVLOWER_NCHW_STRIP_CASE(0)
                CONVLOWER_NCHW_STRIP_CASE(1)
                CONVLOWER_NCHW_STRIP_CASE(2)
                CONVLOWER_NCHW_STRIP_CASE(3)
                CONVLOWER_NCHW_STRIP_CASE(4)
                CONVLOWER_NCHW_STRIP_CASE(5)
                CONVLOWER_NCHW_STRIP_CASE(6)
                CONVLOWER_NCHW_STRIP_CASE(7)
                CONVLOWER_NCHW_STRIP_CASE(8)
                CONVLOWER_NCHW_STRIP_CASE(9)
                default: break;
            }
#undef CONVLOWER_NCHW_STRIP_CASE
        }
        return;
    }
    if (d.kernel == KERN_NCHW_TAPS) {
        if constexpr (sizeof(T) == 4) {
#define CONVLOWER_NCHW_TAPS_CASE(I, S_)                                                                         \
    case I * 16 + S_: {                                                                                         \
        constexpr NchwTapsVariant v = kNchwTapsVariants[I];                                                     \
        GemmArgs h = g;                                                                                         \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                         \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                     \
        conv_nchw_f32_taps_kernel<v.bm, v.bn, v.wgm, v.wgn, v.nbuf, S_><<<blocks, 256, 0, st>>>(h);             \
        break;                                                                                                  \
    }
#define CONVLOWER_NCHW_TAPS_VARIANT(I) CONVLOWER_NCHW_TAPS_CASE(I, 2) CONVLOWER_NCHW_TAPS_CASE(I, 3)
            static_assert(count_of(kNchwTapsVariants) == 6 && count_of(kNchwTapsTaps) == 2 && kNchwTapsTaps[0] == 2 &&
                              kNchwTapsTaps[1] == 3,
                          "compiled filter widths");
            switch (d.variant * 16 + d.p.S) {
                CONVLOWER_NCHW_TAPS_VARIANT(0)
                CONVLOWER_NCHW_TAPS_VARIANT(1)
                CONVLOWER_NCHW_TAPS_VARIANT(2)
                CONVLOWER_NCHW_TAPS_VARIANT(3)
                CONVLOWER_NCHW_TAPS_VARIANT(4)
                CONVLOWER_NCHW_TAPS_VARIANT(5)
                default: break;
            }
#undef CONVLOWER_NCHW_TAPS_VARIANT
#undef CONVLOWER_NCHW_TAPS_CASE
        }
        return;
    }
    if (d.kernel == KERN_STRIP_RB) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_STRIP_RB_CASE(I)                                                                            \
    case I: {                                                                                                 \
        constexpr StripVariant v = kStripRbVariants[I];                                                       \
        GemmArgs h = g;                                                                                       \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                       \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                   \
        conv_strip_rb_kernel<T, v.bm, v.bn, v.wgm, v.wgn, v.strip, v.bst><<<blocks, 64 * v.wgm * v.wgn, 0, st>>>(h); \
        break;                                                                                                \
    }
            switch (d.variant) {
                CONVLOWER_STRIP_RB_CASE(0)
                CONVLOWER_STRIP_RB_CASE(1)
                CONVLOWER_STRIP_RB_CASE(2)
                CONVLOWER_STRIP_RB_CASE(3)
                CONVLOWER_STRIP_RB_CASE(4)
                CONVLOWER_STRIP_RB_CASE(5)
                CONVLOWER_STRIP_RB_CASE(6)
                CONVLOWER_STRIP_RB_CASE(7)
                CONVLOWER_STRIP_RB_CASE(8)
                default: break;
            }
#undef CONVLOWER_STRIP_RB_CASE
        }
        return;
    }
    if (d.kernel == KERN_STRIP_RB2) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_STRIP_RB2_LAUNCH(I, S_)                                                                     \
    case S_: {                                                                                                \
        constexpr StripVariant v = kStripRb2Variants[I];                                                      \
        conv_strip_rb2_kernel<T, v.bm, v.bn, v.wgm, v.wgn, v.strip, S_, v.bst><<<blocks, 64 * v.wgm * v.wgn, 0, st>>>(h); \
        break;                                                                                                \
    }
#define CONVLOWER_STRIP_RB2_CASE(I)                                                                           \
    case I: {                                                                                                 \
        constexpr StripVariant v = kStripRb2Variants[I];                                                      \
        GemmArgs h = g;                                                                                       \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                       \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                   \
        switch (d.p.S) {                                                                                      \
            CONVLOWER_STRIP_RB2_LAUNCH(I, 3)                                                                  \
            CONVLOWER_STRIP_RB2_LAUNCH(I, 5)                                                                  \
            CONVLOWER_STRIP_RB2_LAUNCH(I, 7)                                                                  \
            CONVLOWER_STRIP_RB2_LAUNCH(I, 9)                                                                  \
            CONVLOWER_STRIP_RB2_LAUNCH(I, 11)                                                                 \
            default: break;                                                                                   \
        }                                                                                                     \
        break;                                                                                                \
    }
            switch (d.variant) {
                CONVLOWER_STRIP_RB2_CASE(0)
                CONVLOWER_STRIP_RB2_CASE(1)
                default: break;
            }
#undef CONVLOWER_STRIP_RB2_CASE
#undef CONVLOWER_STRIP_RB2_LAUNCH
        }
        return;
    }
    if (d.kernel == KERN_STRIP_RB3) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_STRIP_RB3_LAUNCH(I, S_)                                                                     \
    case S_: {                                                                                                \
        constexpr StripVariant v = kStripRb3Variants[I];                                                      \
        conv_strip_rb3_kernel<T, v.bm, v.bn, v.wgm, v.wgn, v.strip, S_, v.bst><<<blocks, 64 * v.wgm * v.wgn, 0, st>>>(h); \
        break;                                                                                                \
    }
#define CONVLOWER_STRIP_RB3_CASE(I)                                                                           \
    case I: {                                                                                                 \
        constexpr StripVariant v = kStripRb3Variants[I];                                                      \
        GemmArgs h = g;                                                                                       \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                       \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                   \
        switch (d.p.S) {                                                                                      \
            CONVLOWER_STRIP_RB3_LAUNCH(I, 3)                                                                  \
            CONVLOWER_STRIP_RB3_LAUNCH(I, 5)                                                                  \
            CONVLOWER_STRIP_RB3_LAUNCH(I, 7)                                                                  \
            CONVLOWER_STRIP_RB3_LAUNCH(I, 9)                                                                  \
            CONVLOWER_STRIP_RB3_LAUNCH(I, 11)                                                                 \
            default: break;                                                                                   \
        }                                                                                                     \
        break;                                                                                                \
    }
            static_assert(count_of(kStripRb3Variants) == 3, "compiled variants");
            switch (d.variant) {
                CONVLOWER_STRIP_RB3_CASE(0)
                CONVLOWER_STRIP_RB3_CASE(1)
                CONVLOWER_STRIP_RB3_CASE(2)
                default: break;
            }
#undef CONVLOWER_STRIP_RB3_CASE
#undef CONVLOWER_STRIP_RB3_LAUNCH
        }
        return;
    }
    if (d.kernel == KERN_STREAM1X1) {
        if constexpr (sizeof(T) == 2) {
            // persistent: minb workgroups per CU, at most one 16-pixel block
            // per wave to start with
            auto launch = [&](auto kernel, int minb) {
                const int64_t waves = (d.M + 15) / 16;
                const uint32_t blocks = uint32_t(std::max<int64_t>(
                    1, std::min<int64_t>((waves + 3) / 4, int64_t(minb) * kStreamKCus)));
                kernel<<<blocks, 256, 0, st>>>(g);
            };
#define CONVLOWER_STREAM1X1_CASE(I)                                                                        \
    case I: {                                                                                              \
        constexpr Stream1x1Variant v = kStream1x1Variants[I];                                              \
        if (d.p.C == 32) launch(conv_1x1_stream_kernel<T, 1, v.d, v.minb>, v.minb);                        \
        else if (d.p.C == 64) launch(conv_1x1_stream_kernel<T, 2, v.d, v.minb>, v.minb);                   \
        else if (d.p.C == 128) launch(conv_1x1_stream_kernel<T, 4, v.d, v.minb>, v.minb);                  \
        break;                                                                                             \
    }
            static_assert(count_of(kStream1x1Variants) == 4, "compiled variants");
            switch (d.variant) {
                CONVLOWER_STREAM1X1_CASE(0)
                CONVLOWER_STREAM1X1_CASE(1)
                CONVLOWER_STREAM1X1_CASE(2)
                CONVLOWER_STREAM1X1_CASE(3)
                default: break;
            }
#undef CONVLOWER_STREAM1X1_CASE
        }
        return;
    }
    if (d.kernel == KERN_STRIP_RB4) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_STRIP_RB4_LAUNCH(I, S_)                                                                     \
    case S_: {                                                                                                \
        constexpr StripVariant v = kStripRb4Variants[I];                                                      \
        conv_strip_rb4_kernel<T, v.bm, v.bn, v.wgm, v.wgn, v.strip, S_, (v.bst < S_ ? v.bst : S_),              \
                              kStripRb4Direct[I]>                                                        \
            <<<blocks, 64 * v.wgm * v.wgn, 0, st>>>(h);                                                        \
        break;                                                                                                \
    }
#define CONVLOWER_STRIP_RB4_CASE(I)                                                                           \
    case I: {                                                                                                 \
        constexpr StripVariant v = kStripRb4Variants[I];                                                      \
        GemmArgs h = g;                                                                                       \
        h.tiles_n = int32_t((d.p.K + v.bn - 1) / v.bn);                                                       \
        const uint32_t blocks = uint32_t(((uint64_t(d.M) + v.bm - 1) / v.bm) * h.tiles_n);                   \
        switch (d.p.S) {                                                                                      \
            CONVLOWER_STRIP_RB4_LAUNCH(I, 3)                                                                  \
            CONVLOWER_STRIP_RB4_LAUNCH(I, 5)                                                                  \
            CONVLOWER_STRIP_RB4_LAUNCH(I, 7)                                                                  \
            CONVLOWER_STRIP_RB4_LAUNCH(I, 9)                                                                  \
            CONVLOWER_STRIP_RB4_LAUNCH(I, 11)                                                                 \
            default: break;                                                                                   \
        }                                                                                                     \
        break;                                                                                                \
    }
            static_assert(count_of(kStripRb4Variants) == 5 && count_of(kStripRb4Direct) == 5, "compiled variants");
            switch (d.variant) {
                CONVLOWER_STRIP_RB4_CASE(0)
                CONVLOWER_STRIP_RB4_CASE(1)
                CONVLOWER_STRIP_RB4_CASE(2)
                CONVLOWER_STRIP_RB4_CASE(3)
                CONVLOWER_STRIP_RB4_CASE(4)
                default: break;
            }
#undef CONVLOWER_STRIP_RB4_CASE
#undef CONVLOWER_STRIP_RB4_LAUNCH
        }
        return;
    }
    if (d.kernel == KERN_STRIP) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_STRIP_CASE(I)                                                          \
    case I: {                                                                            \
        constexpr StripVariant v = kStripVariants[I];                                    \
        launch_strip<T, v.bm, v.bn, v.wgm, v.wgn, v.strip, v.bst>(d, g, st); \
        break;                                                                           \
    }
            switch (d.variant) {
                CONVLOWER_STRIP_CASE(0)
                CONVLOWER_STRIP_CASE(1)
                CONVLOWER_STRIP_CASE(2)
                CONVLOWER_STRIP_CASE(3)
                CONVLOWER_STRIP_CASE(4)
                default: break;
            }
#undef CONVLOWER_STRIP_CASE
        }
        return;
    }
    if (d.kernel == KERN_WIDE) {
        if constexpr (sizeof(T) == 2) {
#define CONVLOWER_WIDE_CASE(I)                                                           \
    case I: {                                                                            \
        constexpr TileVariant v = kWideVariants[I];                                      \
        launch_dma_tile<T, v.bm, v.bn, v.bk, v.wgm, v.wgn, v.stages, true>(d, g, st); \
        break;                                                                           \
    }
            switch (d.variant) {
                CONVLOWER_WIDE_CASE(0)
                CONVLOWER_WIDE_CASE(1)
                CONVLOWER_WIDE_CASE(2)
                CONVLOWER_WIDE_CASE(3)
                CONVLOWER_WIDE_CASE(4)
                CONVLOWER_WIDE_CASE(5)
                CONVLOWER_WIDE_CASE(6)
                CONVLOWER_WIDE_CASE(7)
                CONVLOWER_WIDE_CASE(8)
                default: break;
            }
#undef CONVLOWER_WIDE_CASE
            launch_split_reduce<T>(d, g, bias, y, st);
        }
        return;
    }
    switch (d.variant) {
        case 0: launch_gemm_tile<T, 128, 128, 32 / DIV, 2, 2>(d, g, st); break;
        case 1: launch_gemm_tile<T, 128, 64, 32 / DIV, 2, 2>(d, g, st); break;
        default: launch_gemm_tile<T, 128, 32, 32 / DIV, 4, 1>(d, g, st); break;
    }
}

}  // namespace convlower
