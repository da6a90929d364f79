// Library-internal descriptor and kernel tables, shared by the host planner
// (convlower.hip) and the per-dtype contraction launchers (contract_*.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/convlower.h"

// Contraction kernels.
enum KernelId : int32_t {
    KERN_REG = 0,    // register-staged, double-buffered LDS (any A side)
    KERN_DMA = 1,    // LDS-DMA ring, two waves per SIMD (16-byte chunk A sides)
    KERN_WIDE = 2,   // LDS-DMA ring, one wave per SIMD, wide register tiles (16-bit, NHWC windows)
    KERN_NCHW = 3,   // fp32 NCHW windows by 4-byte LDS-DMA
    KERN_STRIP = 4,  // input row strips staged in LDS once per filter row (16-bit, NHWC, C % 32 == 0, S >= 2)
    KERN_STRIP_RB = 5,  // the same strips, filter fragments streamed into registers from a packed copy
    KERN_NCHW_STRIP = 6,  // fp32 NCHW strips (16-byte row loads), register-streamed filter (pad_w == 0, C % 16 == 0)
    KERN_NCHW_TILE = 7,   // fp32 NCHW small windows: input rows staged once per block of output rows, filter in registers
    KERN_TILE16 = 8,      // 16-bit NHWC small windows: the same staging, window rows read as contiguous runs
    KERN_STREAMK = 9,     // the LDS-DMA pipeline (a kDmaVariants shape) in stream-K form: equal contraction
                          // ranges per workgroup of a persistent grid, split tiles summed from workspace slots
    KERN_STRIP_RB2 = 10,  // the register-streamed strips with the taps unrolled (S in kStripRb2Taps, unit
                          // horizontal dilation), padded strip rows read without conflicts
    KERN_NCHW_TAPS = 11,  // fp32 NCHW: per-tap planes of the tile's window elements (4-byte LDS-DMA
                          // gathers), register-streamed filter, taps unrolled (S in kNchwTapsTaps, C % 16 == 0)
    KERN_STRIP_RB3 = 12,  // the unrolled-tap strips on 16x16x32 MFMAs (S in kStripRb2Taps, unit horizontal
                          // dilation), 80-byte strip rows
    KERN_STRIP_RB4 = 13,  // the same with each tap's filter fragments loaded once per workgroup into an LDS ring
    KERN_STREAM1X1 = 14,  // 16-bit NHWC 1x1, unit stride, no padding, C in {32, 64, 128}, K <= 128 and a multiple
                          // of 4: persistent waves streaming 16-pixel blocks through LDS rings, the filter in
                          // registers
};

// One compiled tile shape: BM x BN output tile, BK-deep LDS stages (in 16-bit
// elements; fp32 uses BK/2, the same bytes per row), WGM x WGN waves, STAGES
// LDS stages (0 for the register-staged kernel).  early (pipelined kernel):
// the loads of tile kt+STAGES-1 are issued right after the barrier of tile
// kt, before its MFMAs, instead of after them -- one more tile's MFMA time
// to cover their latency.
struct TileVariant {
    int bm, bn, bk, wgm, wgn, stages, early;
};

constexpr TileVariant kRegVariants[] = {
    {128, 128, 32, 2, 2, 0}, {128, 64, 32, 2, 2, 0}, {128, 32, 32, 4, 1, 0},
};
constexpr TileVariant kDmaVariants[] = {
    {128, 32, 32, 4, 1, 4}, {128, 64, 32, 2, 2, 4}, {128, 128, 32, 2, 2, 4}, {256, 128, 32, 2, 2, 3},
    {256, 128, 32, 4, 2, 4}, {256, 256, 32, 4, 2, 3}, {128, 128, 64, 2, 2, 2}, {128, 128, 64, 4, 2, 2},
    {128, 128, 64, 4, 2, 2, 1}, {128, 128, 64, 2, 2, 2, 1}, {256, 128, 64, 4, 2, 2, 1}, {64, 128, 64, 2, 2, 3, 1},
    {128, 128, 64, 4, 2, 4, 1}, {256, 128, 64, 4, 2, 3, 1},
};
// The pipelined shapes planned for one round of tiles (fewer tiles than CUs;
// 1x1 layers: 256 x 128 tiles): never split, as their point is one tile per CU.
constexpr int kDmaOneRound = 12;
constexpr int kDmaOneRound1x1 = 13;
static_assert(kDmaVariants[kDmaOneRound].bm == 128 && kDmaVariants[kDmaOneRound].stages == 4, "one-round shape");
static_assert(kDmaVariants[kDmaOneRound1x1].bm == 256 && kDmaVariants[kDmaOneRound1x1].stages == 3, "one-round shape");
// The ConvLSTM step's contraction: 64 packed gate rows per tile, one wave
// across them (the cell update needs all four gates of a hidden channel).
constexpr TileVariant kLstmVariant = {128, 64, 32, 4, 1, 4};
constexpr TileVariant kWideVariants[] = {
    {512, 128, 32, 4, 1, 4}, {512, 128, 32, 4, 1, 3}, {256, 256, 32, 2, 2, 3}, {256, 256, 32, 2, 2, 4},
    {256, 128, 32, 2, 2, 4}, {128, 128, 32, 2, 2, 4}, {256, 128, 32, 2, 1, 3}, {256, 128, 64, 2, 2, 3},
    {128, 256, 32, 2, 2, 4},
};
// fp32 NCHW kernel: BK in fp32 elements, 2 x 2 waves except where noted in
// its launcher (BN = 32 uses 4 x 1).
constexpr TileVariant kNchwVariants[] = {
    {128, 32, 32, 4, 1, 3}, {128, 64, 32, 2, 2, 3}, {128, 128, 32, 2, 2, 3}, {64, 128, 32, 2, 2, 3},
    {128, 64, 16, 2, 2, 4}, {128, 64, 16, 2, 2, 6}, {64, 64, 32, 2, 2, 4},  {64, 64, 16, 2, 2, 6},
    {128, 32, 16, 4, 1, 4}, {128, 32, 16, 4, 1, 2}, {64, 32, 16, 4, 1, 2}, {128, 32, 16, 4, 1, 3},
};
// Strip-staged kernel: BM x BN tile, WGM x WGN waves, STRIP 16-byte chunk
// slots per strip buffer (bounds (ceil-ish BM/Q + 1) * W_used * 4), BST
// filter stages.
struct StripVariant {
    int bm, bn, wgm, wgn, strip, bst;
};
constexpr StripVariant kStripVariants[] = {
    {512, 128, 4, 1, 2816, 4}, {256, 128, 2, 2, 1536, 4}, {256, 256, 2, 2, 1536, 4},
    {128, 128, 2, 2, 1024, 4}, {128, 256, 2, 2, 1024, 4},
};
// Strip kernel with register-streamed filter fragments: `bst` is the number
// of steps the filter loads run ahead (DB).
// Unrolled-tap form (conv_strip_rb2_kernel): `strip` counts 16-byte slots of
// padded rows (five per row), `bst` the filter prefetch distance; compiled for
// the filter widths in kStripRb2Taps.
constexpr StripVariant kStripRb2Variants[] = {
    {512, 128, 4, 1, 3584, 2}, {256, 128, 4, 1, 1792, 1},
};
constexpr int kStripRb2Taps[] = {3, 5, 7, 9, 11};
// The 16x16 form: the same padded rows.
// (The filter two steps ahead instead of one measured level or slower on the
// kernel-size layers, with more registers.)
// Variant 2: variant 0's tiles with strip buffers of 48 KiB (eight output
// rows of up to 76 strip rows where Q divides 512).
constexpr StripVariant kStripRb3Variants[] = {
    {512, 128, 4, 1, 3584, 1}, {256, 128, 4, 1, 1792, 1}, {512, 128, 4, 1, 3072, 1}};
// The LDS-shared filter form: bst = how many taps ahead the filter slots are
// loaded, at most S (a ring of bst + 1 slots of BN/16 KiB beside the two strip buffers;
// 80 KiB in all, two workgroups per CU).  Variant 1: strip buffers of 24 KiB
// (four output rows of up to 76 strip rows where Q divides 256) and the
// filter three taps ahead.  Variant 2: 512 x 128 tiles over eight waves, 48 KiB
// strip buffers, the filter three taps ahead (128 KiB, one workgroup per CU);
// variant 3 the same reading the KRSC filter rows, variant 4 variant 1 so.
// The streaming 1x1 kernel: d = pixel blocks in flight per wave, minb =
// workgroups per CU (the persistent grid is minb per CU).
struct Stream1x1Variant {
    int d, minb;
};
constexpr Stream1x1Variant kStream1x1Variants[] = {{3, 2}, {4, 2}, {2, 2}, {4, 1}};   // d * (C/32 + 8) < 64
constexpr StripVariant kStripRb4Variants[] = {
    {256, 128, 4, 1, 1792, 2}, {256, 128, 4, 1, 1536, 3}, {512, 128, 8, 1, 3072, 3}, {512, 128, 8, 1, 3072, 3},
    {256, 128, 4, 1, 1536, 3}};
// Variants that read the caller's KRSC filter rows instead of a packed copy.
constexpr bool kStripRb4Direct[] = {false, false, false, true, true};
constexpr StripVariant kStripRbVariants[] = {
    {512, 128, 4, 1, 2816, 2}, {512, 128, 4, 1, 2816, 3}, {256, 128, 2, 2, 1536, 2},
    {128, 128, 2, 2, 1024, 2}, {256, 256, 2, 2, 1536, 2}, {512, 128, 4, 1, 2816, 4},
    {128, 128, 2, 2, 1024, 4}, {512, 128, 8, 1, 3072, 2}, {256, 128, 4, 1, 1536, 2},
};
// fp32 NCHW strip kernel: strip = 16-byte slots per buffer (16 channel
// planes of ((BM-1)/Q + 2) rows x ceil(W_used/4) slots), db = filter
// prefetch depth in steps, nbuf = strip buffers (strips loaded nbuf-1
// ahead).
struct NchwStripVariant {
    int bm, bn, wgm, wgn, strip, db, nbuf;
};
constexpr NchwStripVariant kNchwStripVariants[] = {
    {128, 64, 2, 2, 1536, 3, 2}, {128, 64, 2, 2, 1536, 4, 3}, {64, 64, 2, 2, 1024, 4, 3},
    {64, 64, 2, 2, 1024, 4, 2},  {64, 128, 2, 2, 1024, 4, 3}, {128, 128, 2, 2, 1536, 2, 2},
    {64, 64, 2, 2, 1024, 6, 3},  {128, 32, 4, 1, 1536, 4, 3}, {64, 32, 4, 1, 1024, 4, 3},
    {64, 64, 4, 1, 1024, 4, 3},
};
// fp32 NCHW tap-plane kernel: BM x BN tiles over wgm x wgn waves, nbuf LDS
// buffers of one (filter row, 16-channel block) each; compiled for the
// filter widths in kNchwTapsTaps.
struct NchwTapsVariant {
    int bm, bn, wgm, wgn, nbuf;
};
constexpr NchwTapsVariant kNchwTapsVariants[] = {
    {128, 64, 2, 2, 2}, {128, 64, 2, 2, 3}, {128, 128, 2, 2, 2}, {64, 64, 2, 2, 2}, {64, 64, 2, 2, 3}, {64, 128, 2, 2, 2},
};
constexpr int kNchwTapsTaps[] = {2, 3};
// LDS bytes of one buffer of the tap-plane kernel: 16 channels x S taps
// planes of nchw_taps_plane(bm, S) words.
constexpr int32_t nchw_taps_plane(int32_t bm, int32_t S) {
    for (int32_t p = bm; p < bm + 64; ++p)
        if ((4 * S * p) % 64 == 16 || (4 * S * p) % 64 == 48) return p;
    return bm;
}
constexpr int64_t nchw_taps_lds(int32_t bm, int32_t S, int32_t nbuf) {
    return int64_t(nbuf) * 16 * S * nchw_taps_plane(bm, S) * 4;
}
constexpr int64_t kNchwTapsLds = 81920;   // two workgroups per CU
// fp32 NCHW small-window kernel: ks 16-deep steps (C*R*S <= 16*ks), tn
// 16-channel blocks (K <= 16*tn).
struct NchwTileVariant {
    int ks, tn;
};
constexpr NchwTileVariant kNchwTileVariants[] = {{1, 2}, {2, 2}, {4, 2}, {1, 4}, {2, 4}, {4, 4}};
// LDS budget of its staged rows, and the workgroups it aims for.
constexpr int64_t kNchwTileLds = 32768;
constexpr int64_t kNchwTileWgs = 1024;
// 16-bit NHWC small-window kernel: ks 32-deep steps (4*ks 8-element chunks
// >= R * cpr), tn 16-channel blocks per wave, split waves per pixel block
// (K <= 16*tn*split).
struct Tile16Variant {
    int ks, tn, split;
};
constexpr Tile16Variant kTile16Variants[] = {{2, 2, 1}, {4, 2, 1}, {6, 2, 1}, {8, 2, 1}, {2, 2, 2}, {4, 2, 2},
                                             {6, 2, 2}, {8, 2, 2}, {2, 4, 1}, {4, 4, 1}, {6, 4, 1}};
// LDS budget of its two staging buffers (three workgroups per CU), the
// tiles (blocks of output rows) it aims for, and the CUs its persistent
// grid covers (tile16_wgs_per_cu workgroups each).
constexpr int64_t kTile16Lds = 40960;
constexpr int64_t kTile16Tiles = 4096;
constexpr int64_t kTile16Cus = 256;
// Slots per channel plane in a strip buffer of `strip` slots: the most that
// fit, rounded to 1 mod 4, so that planes 4 apart (one per lane group) start
// 16 banks apart.
constexpr int32_t nchw_strip_plane(int32_t strip) { return strip / 16 - (strip / 16 - 1) % 4; }
template <class V, int N>
constexpr int count_of(const V (&)[N]) {
    return N;
}

struct conv_desc {
    uint32_t magic;
    conv_params_t p;
    int64_t P, Q, M, Kg, W_used, RCp, Kl;
    int32_t elem, vec;
    bool elided;        // no lowering launch: the contraction reads x (implicit, or 1x1 NHWC unpadded)
    bool pack;          // filter needs packing into ws (lowered contraction order)
    bool frag_pack;     // filter packed into MFMA fragment order in ws (register-streamed kernel)
    bool unpadded;      // fp32 lowered rows of R*C elements, not whole vectors (RCp == R*C)
    uint64_t off_filter, bytes_filter, off_low, bytes_low, ws_bytes;
    uint64_t im2win_bytes, im2col_bytes;
    int32_t kernel;     // KernelId
    int32_t variant;    // index into that kernel's variant table
    int32_t tile_m, tile_n, tile_k;
    int32_t tile_rows;  // fp32 NCHW small-window kernel: output rows per workgroup
    int64_t lstm_cx;    // ConvLSTM step descriptor: input channels taken from x (0: a plain convolution)
    // Split contraction (pipelined DMA kernel): ksplit ranges of the
    // contraction per output tile, fp32 partials [ksplit][M*K] in ws at off_part.
    // Stream-K (KERN_STREAMK): sk_grid workgroups, their sum slots
    // [sk_grid][BM*BN] fp32 then sk_grid flags at off_part (bytes_part in all).
    int32_t ksplit;
    uint64_t off_part, bytes_part;
    int32_t sk_grid;
    int32_t tile_order;   // pipelined kernel: conv_tile_order_t
    // Band lowering (NCHW input, or NHWC with C not a whole number of
    // vectors): output rows (band_g) and output columns (band_cw) per item,
    // staged input rows and columns, LDS row and channel pitch (elements) and
    // tile bytes.  band_items == 0: the element-wise kernel.
    int64_t band_items;
    int32_t band_g, band_cw, band_br, band_tw, band_wl, band_cs, band_lds;
};

namespace convlower {

// Workgroups resident per CU for the stream-K grid, and the CUs it covers.
constexpr int64_t kStreamKCus = 256;
constexpr int64_t kStreamKPerCu = 2;

// Enqueue the contraction (with its fused epilogue) for storage type T.
// epoch: a value no earlier launch used (the stream-K flags).
template <typename T>
void launch_gemm(const conv_desc& d, const void* x, const void* w, const void* bias, void* y, const void* ws,
                 uint32_t epoch, hipStream_t st);

// The contraction of a ConvLSTM step with its cell-update epilogue (fp32).
void launch_lstm_gemm(const conv_desc& d, const void* bias, const void* c_prev, void* h_out, void* c_out,
                      const void* ws, hipStream_t st);

extern template void launch_gemm<float>(const conv_desc&, const void*, const void*, const void*, void*,
                                        const void*, uint32_t, hipStream_t);
extern template void launch_gemm<_Float16>(const conv_desc&, const void*, const void*, const void*, void*,
                                           const void*, uint32_t, hipStream_t);
extern template void launch_gemm<__bf16>(const conv_desc&, const void*, const void*, const void*, void*,
                                         const void*, uint32_t, hipStream_t);

}  // namespace convlower
