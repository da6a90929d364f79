// C ABI of the convolution library: descriptor (plan), validation, and the
// launches of the filter pack, the lowering (im2win / im2col) and the MFMA
// contraction.  Every declaration is in include/convlower.h.
//
// The descriptor is pure host arithmetic (no HIP call), so shapes, workspace
// sizes and error codes can be checked without a GPU.  The launch entry
// points make no allocation and no synchronisation: they validate pointers,
// enqueue kernels on the caller's stream and report launch errors.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "../../include/convlower.h"
#include "dispatch.hpp"
#include "lowering.hpp"

using namespace convlower;

namespace {

constexpr uint32_t kDescMagic = 0x636f6e76u;   // marks a live descriptor
constexpr uint64_t kWsAlign = 256;             // workspace sub-buffer alignment (bytes)
constexpr int kStageLdsBytes = 32 * 1024;      // band lowering: staged tile budget per block
constexpr int64_t kBandItems = 2048;           // band lowering: items to aim for (8 per CU)

}  // namespace

namespace {

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool desc_ok(conv_desc_t d) { return d != nullptr && d->magic == kDescMagic; }

conv_status_t from_hip(hipError_t e) { return e == hipSuccess ? CONV_OK : CONV_ERR_HIP; }

// ---------------------------------------------------------------- planning

// The pipelined tile shape compiled in stream-K form: 128 x 128 over eight
// waves, early issue (variant 8), whose registers (at most 128 per lane with
// the blocked window loader or lowered rows) leave two workgroups per CU.
bool streamk_variant(int v) {
    return v >= 0 && v < count_of(kDmaVariants) && kDmaVariants[v].bm == 128 && kDmaVariants[v].bn == 128 &&
           kDmaVariants[v].early == 1 && kDmaVariants[v].wgm * kDmaVariants[v].wgn == 8 && kDmaVariants[v].stages == 2;
}

// force: "<kernel>:<variant>[:<ksplit>[:<tile order>]]" (conv_create_desc_forced,
// conv_tune), or nullptr for the default choice.  lstm: the ConvLSTM step's
// gate convolution, whose contraction reads whole 16-byte chunks of padded
// lowered rows.
conv_status_t plan(const conv_params_t& p, conv_desc& d, const char* force, bool lstm = false) {
    if (p.N < 0 || p.C <= 0 || p.H <= 0 || p.W <= 0 || p.K <= 0 || p.R <= 0 || p.S <= 0) return CONV_ERR_INVALID_ARG;
    if (p.stride_h <= 0 || p.stride_w <= 0 || p.dil_h <= 0 || p.dil_w <= 0 || p.pad_h < 0 || p.pad_w < 0)
        return CONV_ERR_INVALID_ARG;
    if (p.layout != CONV_NCHW && p.layout != CONV_NHWC) return CONV_ERR_INVALID_ARG;
    if (p.dtype != CONV_F32 && p.dtype != CONV_F16 && p.dtype != CONV_BF16) return CONV_ERR_INVALID_ARG;
    if (p.algo != CONV_ALGO_IM2WIN && p.algo != CONV_ALGO_IM2COL && p.algo != CONV_ALGO_IMPLICIT)
        return CONV_ERR_INVALID_ARG;
    const int64_t lim = (int64_t(1) << 31) - 1;
    if (p.N > lim || p.C > lim || p.H > lim || p.W > lim || p.K > lim || p.R > lim || p.S > lim)
        return CONV_ERR_UNSUPPORTED;

    // Output extents: the number of window positions inside the padded input.
    const int64_t span_h = p.H + 2 * int64_t(p.pad_h) - int64_t(p.dil_h) * (p.R - 1) - 1;
    const int64_t span_w = p.W + 2 * int64_t(p.pad_w) - int64_t(p.dil_w) * (p.S - 1) - 1;
    if (span_h < 0 || span_w < 0) return CONV_ERR_INVALID_ARG;
    d.P = span_h / p.stride_h + 1;
    d.Q = span_w / p.stride_w + 1;

    d.elem = p.dtype == CONV_F32 ? 4 : 2;
    d.vec = 16 / d.elem;
    d.M = p.N * d.P * d.Q;
    d.Kg = p.C * p.R * p.S;
    d.W_used = (d.Q - 1) * p.stride_w + (p.S - 1) * int64_t(p.dil_w) + 1;
    const bool nhwc = p.layout == CONV_NHWC;
    const bool c_vec = p.C % d.vec == 0;
    const bool implicit = p.algo == CONV_ALGO_IMPLICIT;
    // Lowered rows: R*C rounded up to whole 16-byte vectors, so that every
    // lowered row and contraction tile is read with 16-byte loads -- except
    // fp32 windows whose R*C is not a whole number of vectors (the 3-channel
    // first layers), whose lowered buffers are stored unpadded (one window
    // row every R*C elements) and read element by element: padding 9 to 12
    // would cost a third more workspace than the windows themselves
    // ("Enabling Memory-efficient Im2win Convolution ...", abstract: im2win's
    // point is a smaller lowered buffer than im2col's).  Only while the
    // buffer's elements fit 32-bit indices.  (The same row length for every
    // algorithm, so that im2win_bytes describes one layout per shape; only
    // the lowered algorithms use it.)
    d.unpadded = false;
    if (!lstm && p.dtype == CONV_F32 && (p.R * p.C) % d.vec != 0) {
        const int64_t w_el = p.N * d.P * d.W_used * p.R * p.C;
        const int64_t c_el = d.M * p.S * p.R * p.C;
        d.unpadded = w_el < lim && c_el < lim && d.M < lim;
    }
    d.RCp = d.unpadded ? p.R * p.C : int64_t(round_up(uint64_t(p.R * p.C), uint64_t(d.vec)));
    d.Kl = p.S * d.RCp;

    d.elided = implicit || (nhwc && p.R == 1 && p.S == 1 && p.pad_h == 0 && p.pad_w == 0 && c_vec);
    // KRSC with R == 1 or S == 1 is already the (s, r, c) order when C fills whole vectors;
    // the implicit contraction reads the filter in its own order.
    d.pack = !implicit && !(nhwc && c_vec && (p.R == 1 || p.S == 1));

    // 32-bit index ranges used inside the kernels.
    if (d.M > lim || d.Kl > lim || p.K * d.Kl > lim || d.P * d.Q > lim || p.K * d.Kg > lim) return CONV_ERR_UNSUPPORTED;
    if (p.N * d.P > lim || d.W_used * d.RCp > lim) return CONV_ERR_UNSUPPORTED;

    const uint64_t e = uint64_t(d.elem);
    d.im2win_bytes = uint64_t(p.N) * d.P * d.W_used * d.RCp * e;
    d.im2col_bytes = uint64_t(d.M) * d.Kg * e;
    const uint64_t col_bytes = uint64_t(d.M) * d.Kl * e;
    const uint64_t low_vec = (p.algo == CONV_ALGO_IM2WIN ? d.im2win_bytes : col_bytes) / 16;
    if (!d.elided && low_vec > 0x7fffffffull) return CONV_ERR_UNSUPPORTED;
    if (d.P * d.Q > 0 && (d.W_used * d.RCp / d.vec + 255) / 256 > 65535) return CONV_ERR_UNSUPPORTED;

    d.off_filter = 0;
    d.bytes_filter = d.pack ? uint64_t(p.K) * d.Kl * e : 0;
    d.off_low = round_up(d.bytes_filter, kWsAlign);
    d.bytes_low = d.elided ? 0 : (p.algo == CONV_ALGO_IM2WIN ? d.im2win_bytes : col_bytes);
    d.ws_bytes = d.bytes_low ? d.off_low + d.bytes_low : d.bytes_filter;
    if (p.N == 0) d.ws_bytes = 0;

    // Contraction kernel.  The pipelined kernel takes every A side made of
    // whole 16-byte chunks (NHWC windows with C a multiple of the vector, or
    // lowered / in-place rows) while its operand buffers fit 32-bit offsets.
    const uint64_t x_bytes = uint64_t(p.N) * p.C * p.H * p.W * e;
    const uint64_t a_bytes = d.elided ? x_bytes : d.bytes_low;
    const uint64_t b_bytes = uint64_t(p.K) * (implicit ? d.Kg : d.Kl) * e;
    const bool a_chunks = implicit ? (nhwc && c_vec) : !d.unpadded;
    const bool dma_ok = a_chunks && a_bytes < (uint64_t(1) << 31) && b_bytes < (uint64_t(1) << 31);
    // fp32 NCHW fused windows: the pipelined kernel with 4-byte window loads.
    const bool nchw_ok = implicit && !nhwc && p.dtype == CONV_F32 && x_bytes < (uint64_t(1) << 31) &&
                         b_bytes < (uint64_t(1) << 31);
    // 16-bit NHWC windows whose channels fill whole 32-element tile rows: the
    // one-wave-per-SIMD wide-tile kernel.
    const bool wide_ok = dma_ok && implicit && nhwc && p.dtype != CONV_F32 && p.C % 32 == 0;
    // The strip kernel: the same operands, a filter at least two taps wide,
    // and the input rows under a tile's pixels fitting its strip buffer.
    // fp32 NCHW strips: no horizontal padding (rows are loaded from column
    // 0 in 16-byte pieces), 16-channel blocks, and the rows under a tile's
    // pixels fitting the buffer.
    auto nchw_strip_fits = [&](const NchwStripVariant& v) {
        const int64_t rows = (v.bm - 1) / d.Q + 2, wq = (d.W_used + 3) / 4;
        return nchw_ok && p.pad_w == 0 && p.C % 16 == 0 &&
               uint64_t((p.K + 15) / 16 * 16) * d.Kg * 4 < (uint64_t(1) << 31) && rows < 256 && wq < 256 &&
               rows * wq <= nchw_strip_plane(v.strip);
    };
    // fp32 NCHW tap planes: a compiled filter width, 16-channel blocks, and
    // the buffers of two workgroups within a CU's LDS.
    auto nchw_taps_fits = [&](const NchwTapsVariant& v) {
        bool taps = false;
        for (int t : kNchwTapsTaps) taps = taps || p.S == t;
        return nchw_ok && taps && p.C % 16 == 0 &&
               uint64_t((p.K + 15) / 16 * 16) * d.Kg * 4 < (uint64_t(1) << 31) &&
               nchw_taps_lds(v.bm, int32_t(p.S), v.nbuf) <= kNchwTapsLds;
    };
    // fp32 NCHW small windows (C*R*S <= 64, K <= 64): output rows per
    // workgroup so that there are about kNchwTileWgs workgroups and a
    // block's staged input rows fit kNchwTileLds; 0 where it does not apply.
    auto nchw_tile_rows = [&](const NchwTileVariant& v) -> int64_t {
        if (!nchw_ok || d.Kg > 16 * v.ks || p.K > 16 * v.tn) return 0;
        const int64_t row_bytes = (p.C + 1) * d.W_used * 4;   // C planes and a zero plane
        const int64_t fit_rows = (kNchwTileLds - 1024 * v.tn * v.ks - 64 * v.tn - 16) / row_bytes - (p.R - 1) * int64_t(p.dil_h) - 1;
        if (fit_rows < 0) return 0;
        const int64_t tmax = fit_rows / p.stride_h + 1;
        const int64_t per_img = (kNchwTileWgs + p.N - 1) / p.N;
        const int64_t tp = (d.P + per_img - 1) / per_img;
        return tp < tmax ? tp : tmax;
    };
    auto strip_fits = [&](const StripVariant& v) {
        const int64_t rows = (v.bm - 1) / d.Q + 2;
        return wide_ok && p.S >= 2 && rows * d.W_used * 4 <= v.strip;
    };
    // The unrolled-tap strip kernel: a compiled filter width, unit
    // horizontal dilation, and the padded rows (five slots each) fitting.
    auto strip2_fits = [&](const StripVariant& v) {
        bool taps = false;
        for (int t : kStripRb2Taps) taps = taps || p.S == t;
        // output rows a tile touches: bm / Q where Q divides bm (tiles start
        // on a row), else at most (bm - 1) / Q + 2
        const int64_t rows = v.bm % d.Q == 0 ? v.bm / d.Q : (v.bm - 1) / d.Q + 2;
        return wide_ok && taps && p.dil_w == 1 && rows * d.W_used * 5 <= v.strip;
    };
    // Its 16x16 form: the same.
    auto strip3_fits = [&](const StripVariant& v) { return strip2_fits(v); };
    // 16-bit NHWC small windows: unit horizontal dilation, every staged
    // word and window run 4-byte aligned ((C*sw) and (W*C) even), a window
    // row of at most 256 elements, and one image within 32-bit offsets.
    const bool tile16_ok = implicit && nhwc && p.dtype != CONV_F32 && p.dil_w == 1 &&
                           (p.C * int64_t(p.stride_w)) % 2 == 0 && (p.W * int64_t(p.C)) % 2 == 0 &&
                           p.S * int64_t(p.C) <= 256 && p.pad_w <= 65536 &&
                           uint64_t(p.C) * p.H * p.W * e < (uint64_t(1) << 31);
    // The streaming 1x1 kernel: unit stride and no padding make x the
    // pixel-row matrix itself; its whole filter fits one LDS fragment copy.
    const bool stream1x1_ok = p.dtype != CONV_F32 && nhwc && d.elided && p.R == 1 && p.S == 1 &&
                              p.stride_h == 1 && p.stride_w == 1 && p.pad_h == 0 && p.pad_w == 0 &&
                              (p.C == 32 || p.C == 64 || p.C == 128) && p.K <= 128 && p.K % 4 == 0 &&
                              x_bytes < (uint64_t(1) << 31) && uint64_t(d.M) * p.K * e < (uint64_t(1) << 31);
    // Its output rows per tile for a variant (the window rows in at most
    // 4*ks chunks, K <= 16*tn*split): about kTile16Tiles tiles, two tiles' staged
    // rows within kTile16Lds; 0 where it does not apply.
    auto tile16_rows = [&](const Tile16Variant& v) -> int64_t {
        if (!tile16_ok || p.K > 16 * v.tn * v.split) return 0;
        const Tile16Geom geo = tile16_geom(int(p.C), int(p.S), int(p.pad_w));
        if (p.R * int64_t(geo.cpr) > 4 * v.ks) return 0;
        const int64_t row_bytes = ((d.Q - 1) * p.stride_w * p.C + 8 * geo.cpr) * 2;
        const int64_t fit_rows = kTile16Lds / 2 / row_bytes - (p.R - 1) * int64_t(p.dil_h) - 1;
        if (fit_rows < 0) return 0;
        const int64_t tmax = fit_rows / p.stride_h + 1;
        const int64_t per_img = (kTile16Tiles + p.N - 1) / p.N;
        const int64_t tp = (d.P + per_img - 1) / per_img;
        return tp < tmax ? tp : tmax;
    };
    if (nchw_ok) {
        // fp32 NCHW: narrow K -> 128-row tiles, 16-deep stages; wide K ->
        // 64-row tiles, 64 or 128 channels wide depending on how many
        // workgroups that gives.
        d.kernel = KERN_NCHW;
        if (p.K <= 32)
            d.variant = d.Kg <= 32 ? 9 : 8;   // a contraction of one or two tiles: two stages leave room for more workgroups
        else if (p.K <= 64)
            d.variant = 4;
        else
            d.variant = (d.M / 64) * ((p.K + 127) / 128) >= 768 ? 3 : 7;
        // Unpadded rows, 16-channel blocks and taps sharing a row: the strip
        // kernel (a sweep over the encoder's strided layers put it ahead):
        // 128 x 64 tiles up to 64 output channels, else 128 x 128 while that
        // still gives about two tiles per CU, else 64 x 64.
        if (p.S >= 2) {
            const int v = p.K <= 64 ? 0 : ((d.M / 128) * ((p.K + 127) / 128) >= 384 ? 5 : 3);
            if (nchw_strip_fits(kNchwStripVariants[v])) {
                d.kernel = KERN_NCHW_STRIP;
                d.variant = v;
            }
        }
        // Filter widths 2 and 3 that the strip kernel does not take (padded
        // columns), and width 2: the tap-plane kernel, 64 x 64 tiles, or
        // 64 x 128 while that still gives about 1.5 tiles per CU.  Measured
        // cold against the pipelined kernel on padded 3x3 layers it ran 1.1
        // to 1.45 times faster (the 128-channel layer at 28x28 1.9 times
        // faster than the pipelined kernel's default tile for it); on the
        // encoder's 2x2 64->128 layer 7 % faster than the strip kernel, on
        // its 2x2 128->256 layer within 3 %.  On the encoder's 3x3 stride-2
        // layer the strip kernel stays 14 % ahead: its 16-byte row loads
        // move the window with a quarter of the load instructions, which
        // counts once the input comes from HBM.
        if (p.S >= 2 && !(p.S == 3 && d.kernel == KERN_NCHW_STRIP)) {
            const int tv = p.K <= 64 ? 3 : ((d.M / 64) * ((p.K + 127) / 128) >= 384 ? 5 : 3);
            if (nchw_taps_fits(kNchwTapsVariants[tv])) {
                d.kernel = KERN_NCHW_TAPS;
                d.variant = tv;
            }
        }
        // Small windows and few output channels: the whole filter in
        // registers and the input rows staged once per block of output rows.
        if (d.Kg <= 64 && p.K <= 64) {
            const int v = (d.Kg <= 16 ? 0 : d.Kg <= 32 ? 1 : 2) + (p.K <= 32 ? 0 : 3);
            if (nchw_tile_rows(kNchwTileVariants[v]) > 0) {
                d.kernel = KERN_NCHW_TILE;
                d.variant = v;
            }
        }
    } else if (dma_ok) {
        // BN covers the output channels up to 128.  fp32: BM = 256 where that
        // still gives two workgroups per CU, else 128.  16-bit: 128 x 128
        // tiles over eight waves with two 64-deep stages, the next tile's
        // loads issued before the MFMAs of the current one -- ahead of the
        // same tile issuing after them (5-15 %), of three and four stages
        // (their LDS leaves room for one workgroup per CU instead of two)
        // and of 256 x 128 tiles, on the 3x3, 1x1 and kernel-size layers.
        d.kernel = KERN_DMA;
        d.variant = p.K <= 32 ? 0 : (p.K <= 64 ? 1 : (p.dtype == CONV_F32 ? 2 : 8));
        if (d.variant == 2 && (d.M / 256) * ((p.K + 127) / 128) >= 512) d.variant = 3;
        // 16-bit 1x1 layers with at least two 256 x 128 tiles per CU: those
        // tiles with three 32-deep stages (a short contraction streamed in
        // more, smaller pieces; interleaved timing on the kernel-size sweep's
        // 1x1 layer: 11 % faster than the 128 x 128 default)
        if (d.variant == 8 && p.R == 1 && p.S == 1 && (d.M / 256) * ((p.K + 127) / 128) >= 512) d.variant = 3;
        // Fewer 128 x 128 tiles than CUs: 1x1 layers, 128 x 128 over four
        // waves (the 1x1 1024-channel layer at 14x14: 2-7 % ahead of the
        // eight-wave tiles, conv_tune's pick) -- or, with 128 to 255 tiles
        // of 256 x 128, those in one round, over eight waves with three
        // 64-deep stages (144 KiB of LDS; that layer, 196 such tiles: 8 %
        // faster cold than the four-wave 128 x 128 tiles, 5 % ahead of
        // 128 x 256 tiles).  Otherwise, from half as many tiles as CUs, one round of
        // 128 x 128 tiles over eight waves with four 64-deep stages (128 KiB
        // of LDS, one workgroup per CU): cold, 2-3 % faster than the 64 x 128
        // tiles below on the 3x3 256-channel layer at 14x14 and the 3x3
        // 512-channel layer at 7x7 (both 196 tiles), 20 % faster than the
        // same tiles with two stages; five stages level, six or eight 32-deep
        // ones 15-24 % slower.  Below that, 64 x 128 tiles over four waves
        // (twice the workgroups) with three 64-deep stages (two workgroups
        // per CU fit; on the 3x3 256-channel layer at 14x14 6 % faster cold
        // than the 128 x 128 two-stage tiles, another 9 % with the third
        // stage).
        const int64_t tiles128 = (d.M / 128) * ((p.K + 127) / 128);
        const int64_t tiles256 = (d.M / 256) * ((p.K + 127) / 128);
        if (d.variant == 8 && p.R == 1 && p.S == 1)
            d.variant = tiles256 >= 128 && tiles256 < 256 ? kDmaOneRound1x1 : 9;
        else if (d.variant == 8 && tiles128 < 256)
            d.variant = tiles128 >= 128 ? kDmaOneRound : 11;
        // 1x1 layers the streaming kernel takes, from 16384 pixels: it
        // (C = K = 128 at 64x64, by interleaved timing after a 512 MiB
        // read-modify-write pass: 13 % faster than the 256 x 128 tiles at 32
        // images, 21 % at 128; 13 % faster than 128 x 128 tiles at 8 images)
        // -- two workgroups per CU with two blocks in flight per wave below
        // 131072 pixels, one with four from there.
        if (stream1x1_ok && d.M >= 16384) {
            d.kernel = KERN_STREAM1X1;
            d.variant = d.M >= 131072 ? 3 : 2;
        }
        // 3x3 with at least two 256 x 128 strip tiles per CU: the unrolled-tap
        // strips on 16x16x32 MFMAs, 256 x 128 tiles (conv_tune's pick on the
        // kernel-size sweep's 3x3 layer, 12 % faster than the pipelined tiles).
        if (p.S == 3 && p.K % 128 == 0 && (d.M / 256) * (p.K / 128) >= 512 && strip3_fits(kStripRb3Variants[1])) {
            d.kernel = KERN_STRIP_RB3;
            d.variant = 1;
        }
        // Filter rows of 5 taps and more, enough strip tiles to give most CUs
        // one, and output channels filling whole 128-wide tiles: the
        // register-streamed strip kernel (interleaved timing on the
        // kernel-size layers: ahead of the pipelined tiles by 3 % at 5 x 5,
        // 3 % at 7 x 7 and a quarter at 11 x 11, behind by 15 % at 3 x 3).
        // From 9 taps 512 x 128 tiles over four waves, one per SIMD, the
        // filter prefetch 4 steps ahead; below, 256 x 128 tiles whose 64 x 128
        // wave tiles leave room for two waves per SIMD (level at 11 x 11, 3 %
        // ahead at 5 x 5 and 7 x 7).
        // Where the filter width is one the unrolled-tap form is compiled for
        // and the horizontal dilation is 1, that form (512 x 128 tiles, the
        // filter 2 steps ahead): interleaved timing on the kernel-size layers,
        // 12 % faster than the general strip kernel at 11 x 11, 9 % at 7 x 7,
        // 6 % at 5 x 5.
        const int rbv = p.S >= 9 ? 5 : 8;
        const StripVariant& rb = kStripRbVariants[rbv];
        if (p.S >= 5 && p.K % 128 == 0 && (d.M / rb.bm) * (p.K / rb.bn) >= 192 && strip_fits(rb)) {
            d.kernel = KERN_STRIP_RB;
            d.variant = rbv;
            const StripVariant& rb2 = kStripRb2Variants[0];
            if ((d.M / rb2.bm) * (p.K / rb2.bn) >= 192 && strip2_fits(rb2)) {
                d.kernel = KERN_STRIP_RB2;
                d.variant = 0;
                // Its 16x16x32 form (the same tiles, the filter one step
                // ahead): 5-8 % faster on the 5x5 to 11x11 layers, where the
                // shader clock holds higher under the 16x16 instruction.
                if (strip3_fits(kStripRb3Variants[0])) {
                    d.kernel = KERN_STRIP_RB3;
                    d.variant = 0;
                    // the same tiles with a strip buffer cut to what the rows
                    // need where they fit it (two fewer strip loads a lane;
                    // about 1 % at 9 x 9 and 11 x 11)
                    if (strip3_fits(kStripRb3Variants[2])) d.variant = 2;
                }
            }
        }
        // Up to 7 taps, with at least two 256 x 128 strip tiles per CU: the
        // same strips with the filter shared through LDS, two workgroups per
        // CU (interleaved timing on the kernel-size layers: 5 % faster at
        // 3 x 3 and 5 x 5, 1 % at 7 x 7; 1 % and 3 % slower at 9 x 9 and
        // 11 x 11, which keep the 512 x 128 tiles).  Where the rows fit the
        // smaller strip buffers, those with the filter three taps ahead
        // (another 3 % at 3 x 3, 1 % at 5 x 5 and 7 x 7).
        if ((p.S == 3 || p.S == 5 || p.S == 7) && p.K % 128 == 0 && (d.M / 256) * (p.K / 128) >= 512 &&
            (d.kernel == KERN_STRIP_RB3 || d.kernel == KERN_STRIP_RB2) && strip3_fits(kStripRb4Variants[0])) {
            d.kernel = KERN_STRIP_RB4;
            d.variant = strip3_fits(kStripRb4Variants[1]) ? 1 : 0;
        }
        // Where either strip form was chosen and there are enough 512 x 128
        // tiles to give most CUs one: those tiles over eight waves (two per
        // SIMD, one workgroup per CU) with the filter shared through LDS --
        // one filter load per wave and tap instead of two, and 8 instead of
        // 32 per workgroup in the register form (interleaved timing: 2-3 %
        // faster from 7 x 7 to 11 x 11 than both).  Up to 7 taps reading the
        // caller's KRSC filter rows, which saves the packing pass (with it, 6 %
        // faster than the 256 x 128 tiles at 3 x 3 and 3 % at 5 x 5, 1 % at
        // 7 x 7); from 9 taps the packed copy (level at 9 x 9, and at 11 x 11
        // 1 % faster after a cache flush, pass included).
        if ((d.kernel == KERN_STRIP_RB3 || d.kernel == KERN_STRIP_RB4) && (d.M / 512) * (p.K / 128) >= 192 &&
            strip3_fits(kStripRb4Variants[3])) {
            d.kernel = KERN_STRIP_RB4;
            d.variant = p.S <= 7 ? 3 : 2;
        }
    } else {
        d.kernel = KERN_REG;
        d.variant = p.K <= 32 ? 2 : (p.K <= 64 ? 1 : 0);
    }
    // 16-bit NHWC windows of channels that do not fill whole vectors (the
    // stem layers) into at most 64 output channels: the small-window kernel
    // with the fewest steps that cover its chunks.
    if (tile16_ok && !dma_ok && p.K <= 64) {
        // K <= 32: two channel blocks per wave; else four (one wave per pixel block)
        const int tn = p.K <= 32 ? 2 : 4;
        for (int i = 0; i < count_of(kTile16Variants); ++i)
            if (kTile16Variants[i].tn == tn && kTile16Variants[i].split == 1 && tile16_rows(kTile16Variants[i]) > 0) {
                d.kernel = KERN_TILE16;
                d.variant = i;
                break;
            }
    }
    // Forced choice "<kernel>:<variant>[:<ksplit>]" with kernel one of the
    // names in kKernelFamilies, applied where that kernel takes this
    // convolution (ksplit: the pipelined DMA kernel's contraction split).
    // Stream-K operands: lowered rows, or windows of whole stage-deep channel
    // blocks (the blocked loader; the other one needs more registers than two
    // workgroups per CU allow).
    auto sk_operands = [&](int v) {
        const int64_t bk = p.dtype == CONV_F32 ? kDmaVariants[v].bk / 2 : kDmaVariants[v].bk;
        return !implicit || p.C % bk == 0;
    };
    int force_ks = 0;
    int force_order = -1;
    if (const char* v = force) {
        const char* colon = std::strchr(v, ':');
        if (colon) {
            const std::string name(v, colon - v);
            const int i = std::atoi(colon + 1);
            if (const char* c2 = std::strchr(colon + 1, ':')) {
                force_ks = std::atoi(c2 + 1);
                if (const char* c3 = std::strchr(c2 + 1, ':')) force_order = std::atoi(c3 + 1);
            }
            if (name == "reg" && !nchw_ok && i >= 0 && i < count_of(kRegVariants)) {
                d.kernel = KERN_REG;
                d.variant = i;
            } else if (name == "dma" && dma_ok && !nchw_ok && i >= 0 && i < count_of(kDmaVariants)) {
                d.kernel = KERN_DMA;
                d.variant = i;
            } else if (name == "wide" && wide_ok && i >= 0 && i < count_of(kWideVariants) &&
                       p.C % kWideVariants[i].bk == 0) {
                d.kernel = KERN_WIDE;
                d.variant = i;
            } else if (name == "strip" && i >= 0 && i < count_of(kStripVariants) && strip_fits(kStripVariants[i])) {
                d.kernel = KERN_STRIP;
                d.variant = i;
            } else if (name == "striprb" && i >= 0 && i < count_of(kStripRbVariants) &&
                       strip_fits(kStripRbVariants[i])) {
                d.kernel = KERN_STRIP_RB;
                d.variant = i;
            } else if (name == "striprb2" && i >= 0 && i < count_of(kStripRb2Variants) &&
                       strip2_fits(kStripRb2Variants[i])) {
                d.kernel = KERN_STRIP_RB2;
                d.variant = i;
            } else if (name == "nchwtile" && i >= 0 && i < count_of(kNchwTileVariants) &&
                       nchw_tile_rows(kNchwTileVariants[i]) > 0) {
                d.kernel = KERN_NCHW_TILE;
                d.variant = i;
            } else if (name == "nchwstrip" && i >= 0 && i < count_of(kNchwStripVariants) &&
                       nchw_strip_fits(kNchwStripVariants[i])) {
                d.kernel = KERN_NCHW_STRIP;
                d.variant = i;
            } else if (name == "striprb3" && i >= 0 && i < count_of(kStripRb3Variants) &&
                       strip3_fits(kStripRb3Variants[i])) {
                d.kernel = KERN_STRIP_RB3;
                d.variant = i;
            } else if (name == "stream1x1" && stream1x1_ok && i >= 0 && i < count_of(kStream1x1Variants)) {
                d.kernel = KERN_STREAM1X1;
                d.variant = i;
            } else if (name == "striprb4" && i >= 0 && i < count_of(kStripRb4Variants) &&
                       strip3_fits(kStripRb4Variants[i])) {
                d.kernel = KERN_STRIP_RB4;
                d.variant = i;
            } else if (name == "nchwtaps" && i >= 0 && i < count_of(kNchwTapsVariants) &&
                       nchw_taps_fits(kNchwTapsVariants[i])) {
                d.kernel = KERN_NCHW_TAPS;
                d.variant = i;
            } else if (name == "tile16" && i >= 0 && i < count_of(kTile16Variants) &&
                       tile16_rows(kTile16Variants[i]) > 0) {
                d.kernel = KERN_TILE16;
                d.variant = i;
            } else if (name == "nchw" && nchw_ok && i >= 0 && i < count_of(kNchwVariants)) {
                d.kernel = KERN_NCHW;
                d.variant = i;
            } else if (name == "streamk" && dma_ok && !nchw_ok && streamk_variant(i) && sk_operands(i)) {
                d.kernel = KERN_STREAMK;
                d.variant = i;
            }
        }
    }
    // Split contraction for the pipelined DMA kernel, in two: when the
    // output tiles leave three CUs in four idle (at most 64 of them) or the
    // contraction is very long (4096 elements and more) while there are fewer
    // tiles than CUs, and the contraction has at least 16 tiles.  A
    // sweep over 3x3 and 1x1 layers found more splits, or splits with ~100
    // tiles and shorter contractions, slower than none: the fp32 partials
    // cost a write and a read of ksplit*M*K*4 bytes.  Every split non-empty.
    // (The wide-tile kernel splits only when forced, or when conv_tune keeps
    // such a plan.)
    // Stream-K (the 128 x 128 pipelined tiles over a persistent grid of two
    // workgroups per CU, every workgroup the same share of (tile, step)
    // pairs) is taken only when forced or kept by conv_tune: on the layers
    // whose tiles fill the GPU unevenly (3x3 at 14x14 with 256 channels, 1x1
    // with 1024 input channels) it measured 1.3 to 1.45 times slower than one
    // workgroup per tile.  Its rate on evenly divided layers matches the
    // plain kernel, so the loss is in the split tiles: the pieces of a tile
    // run at different contraction offsets at once and no longer share the
    // window rows they read through L2.
    const auto sk_shape = [&](int v, int64_t& tiles, int64_t& nkt) {
        const TileVariant& tv = kDmaVariants[v];
        const int64_t bk = p.dtype == CONV_F32 ? tv.bk / 2 : tv.bk;
        tiles = ((d.M + tv.bm - 1) / tv.bm) * ((p.K + tv.bn - 1) / tv.bn);
        nkt = ((implicit ? d.Kg : d.Kl) + bk - 1) / bk;
    };
    const int64_t sk_cap = kStreamKCus * kStreamKPerCu;
    d.sk_grid = 0;
    if (d.kernel == KERN_STREAMK) {
        int64_t tiles = 0, nkt = 0;
        sk_shape(d.variant, tiles, nkt);
        d.sk_grid = int32_t(std::max<int64_t>(1, std::min<int64_t>(tiles * nkt, sk_cap)));
    }
    d.ksplit = 1;
    if (d.kernel == KERN_DMA || d.kernel == KERN_WIDE) {
        const TileVariant& tv = d.kernel == KERN_DMA ? kDmaVariants[d.variant] : kWideVariants[d.variant];
        const int64_t bk = p.dtype == CONV_F32 ? tv.bk / 2 : tv.bk;
        const int64_t kc = implicit ? d.Kg : d.Kl;
        const int64_t nkt = (kc + bk - 1) / bk;
        const int64_t tiles = ((d.M + tv.bm - 1) / tv.bm) * ((p.K + tv.bn - 1) / tv.bn);
        int64_t ks = 1;
        if (force_ks > 0) {
            ks = force_ks < 8 ? force_ks : 8;
        } else if (d.kernel == KERN_DMA && d.variant != kDmaOneRound && d.variant != kDmaOneRound1x1 && tiles > 0 && tiles < 256 && nkt >= 16 &&
                   (tiles <= 64 || kc >= 4096)) {
            ks = 2;
        }
        if (ks > nkt) ks = nkt;
        while (ks > 1 && (ks - 1) * ((nkt + ks - 1) / ks) >= nkt) --ks;
        d.ksplit = int32_t(ks < 1 ? 1 : ks);
    }
    // Tile order of the pipelined kernel (the other kernels have their own
    // fixed orders): XCD ranges in serpentine order.  Measured against the
    // plain order: the 3x3 512-channel layer at 7x7 fetched 5.6 times fewer
    // bytes from beyond L2 (31 against 176 MiB per launch) and ran 3 % faster,
    // the 1x1 1024-channel layer 3 % faster, the other 3x3 and 5x5 layers
    // level; column-major ranges were level or slower.  The one-round
    // 128 x 128 tiles take column-major ranges (each XCD's tiles share fewer
    // filter columns): up to 2 % faster cold than serpentine on the 3x3 256-
    // and 512-channel layers at 14x14 and 7x7 (never slower in three
    // interleaved runs); the 256 x 128 one-round tiles on
    // the 1x1 layer stay serpentine (2 % ahead of column-major).
    d.tile_order = d.kernel != KERN_DMA               ? CONV_TILE_LINEAR
                   : d.variant == kDmaOneRound ? CONV_TILE_XCD_COLS
                                                      : CONV_TILE_XCD_SERPENT;
    if (d.kernel == KERN_DMA && force_order >= 0 && force_order <= CONV_TILE_XCD_COLS) d.tile_order = force_order;

    d.tile_rows = 0;
    if (d.kernel == KERN_NCHW_TILE) {
        d.tile_rows = int32_t(nchw_tile_rows(kNchwTileVariants[d.variant]));
        d.tile_m = 16;
        d.tile_n = 16 * kNchwTileVariants[d.variant].tn;
        d.tile_k = 16 * kNchwTileVariants[d.variant].ks;
    } else if (d.kernel == KERN_TILE16) {
        d.tile_rows = int32_t(tile16_rows(kTile16Variants[d.variant]));
        d.tile_m = 16;
        d.tile_n = 16 * kTile16Variants[d.variant].tn * kTile16Variants[d.variant].split;
        d.tile_k = 32 * kTile16Variants[d.variant].ks;
    } else if (d.kernel == KERN_NCHW_STRIP) {
        d.tile_m = kNchwStripVariants[d.variant].bm;
        d.tile_n = kNchwStripVariants[d.variant].bn;
        d.tile_k = 16;
    } else if (d.kernel == KERN_STREAM1X1) {
        d.tile_m = 16;
        d.tile_n = 128;
        d.tile_k = 32;
    } else if (d.kernel == KERN_NCHW_TAPS) {
        d.tile_m = kNchwTapsVariants[d.variant].bm;
        d.tile_n = kNchwTapsVariants[d.variant].bn;
        d.tile_k = 16;
    } else if (d.kernel == KERN_STRIP || d.kernel == KERN_STRIP_RB || d.kernel == KERN_STRIP_RB2 ||
               d.kernel == KERN_STRIP_RB3 || d.kernel == KERN_STRIP_RB4) {
        const StripVariant& sv = d.kernel == KERN_STRIP       ? kStripVariants[d.variant]
                                 : d.kernel == KERN_STRIP_RB  ? kStripRbVariants[d.variant]
                                 : d.kernel == KERN_STRIP_RB2 ? kStripRb2Variants[d.variant]
                                 : d.kernel == KERN_STRIP_RB3 ? kStripRb3Variants[d.variant]
                                                              : kStripRb4Variants[d.variant];
        d.tile_m = sv.bm;
        d.tile_n = sv.bn;
        d.tile_k = 32;
    } else {
        const TileVariant& tv = d.kernel == KERN_NCHW                            ? kNchwVariants[d.variant]
                                : d.kernel == KERN_WIDE                          ? kWideVariants[d.variant]
                                : d.kernel == KERN_DMA || d.kernel == KERN_STREAMK ? kDmaVariants[d.variant]
                                                                                   : kRegVariants[d.variant];
        d.tile_m = tv.bm;
        d.tile_n = tv.bn;
        d.tile_k = d.kernel == KERN_NCHW ? tv.bk : (p.dtype == CONV_F32 ? tv.bk / 2 : tv.bk);
    }

    // The register-streamed strip kernel reads the filter from a copy in MFMA
    // fragment order: output channels padded to a multiple of 32.
    // The small-window kernel's copy: one 16-byte A fragment per lane, 32-deep
    // step and 16-channel block.
    d.frag_pack = d.kernel == KERN_STRIP_RB || d.kernel == KERN_STRIP_RB2 || d.kernel == KERN_STRIP_RB3 ||
                  (d.kernel == KERN_STRIP_RB4 && !kStripRb4Direct[d.variant]) ||
                  d.kernel == KERN_NCHW_STRIP || d.kernel == KERN_NCHW_TAPS || d.kernel == KERN_TILE16;
    if (d.frag_pack) {
        const int64_t kpad =
            d.kernel == KERN_STRIP_RB || d.kernel == KERN_STRIP_RB2 ? (p.K + 31) / 32 * 32 : (p.K + 15) / 16 * 16;
        d.off_filter = 0;
        d.bytes_filter = d.kernel == KERN_TILE16
                             ? uint64_t(1024) * kTile16Variants[d.variant].tn * kTile16Variants[d.variant].split *
                                   kTile16Variants[d.variant].ks
                             : uint64_t(kpad) * d.Kg * e;
        d.ws_bytes = p.N == 0 ? 0 : d.bytes_filter;
    }

    // The split contraction's fp32 partials, or the stream-K sum slots and
    // their flags, go last in the workspace.
    d.off_part = 0;
    d.bytes_part = d.ksplit > 1 ? uint64_t(d.ksplit) * uint64_t(d.M) * uint64_t(p.K) * 4 : 0;
    if (d.kernel == KERN_STREAMK)
        d.bytes_part = uint64_t(d.sk_grid) * uint64_t(d.tile_m) * uint64_t(d.tile_n) * 4 + uint64_t(d.sk_grid) * 4;
    if (d.bytes_part && p.N > 0) {
        d.off_part = round_up(d.ws_bytes, kWsAlign);
        d.ws_bytes = d.off_part + d.bytes_part;
    }

    // Band lowering: the most output rows per item whose staged tile fits
    // kStageLdsBytes, at most P / ceil(kBandItems / N) rows so that the grid
    // has about kBandItems items; when one full-width row does not fit
    // (NCHW), one row and the most output columns that fit.
    d.band_items = 0;
    d.band_g = d.band_cw = d.band_br = d.band_tw = d.band_wl = d.band_cs = d.band_lds = 0;
    if ((!nhwc || !c_vec) && !d.elided && !d.unpadded && p.N > 0 && d.P > 0 && d.Q > 0) {
        const bool win = p.algo == CONV_ALGO_IM2WIN;
        const int64_t full = win ? d.W_used : d.Q;
        const int64_t span = (p.S - 1) * int64_t(p.dil_w) + 1;
        auto tw_of = [&](int64_t cw) { return win ? cw : (cw - 1) * p.stride_w + span; };
        auto br_of = [&](int64_t g) { return (g - 1) * p.stride_h + (p.R - 1) * int64_t(p.dil_h) + 1; };
        // NCHW rows get an odd pitch, which spreads a wave's column reads over banks.
        auto wl_of = [&](int64_t cw) { return nhwc ? p.W * p.C : (tw_of(cw) | 1); };
        // NCHW channel pitch: odd too, or a wave reading every 4th channel meets few banks.
        auto cs_of = [&](int64_t g, int64_t cw) { return nhwc ? br_of(g) * wl_of(cw) : (br_of(g) * wl_of(cw)) | 1; };
        auto lds_of = [&](int64_t g, int64_t cw) { return (nhwc ? 1 : p.C) * cs_of(g, cw) * int64_t(d.elem); };
        const int64_t bands_wanted = (kBandItems + p.N - 1) / p.N;
        const int64_t g_cap = bands_wanted > 1 ? std::max<int64_t>(1, d.P / bands_wanted) : d.P;
        int64_t g = 0, cw = full;
        if (lds_of(1, full) <= kStageLdsBytes) {
            g = 1;
            while (g < g_cap && lds_of(g + 1, full) <= kStageLdsBytes) ++g;
        } else if (!nhwc) {
            // (tw | 1) <= max_wl keeps C * ((br * wl) | 1) within the budget
            const int64_t max_wl = (kStageLdsBytes / (p.C * int64_t(d.elem)) - 1) / br_of(1);
            cw = win ? max_wl - 1 : (max_wl - 1 - span) / p.stride_w + 1;
            if (max_wl >= 2 && cw >= 1 && tw_of(cw) >= 1 && lds_of(1, cw) <= kStageLdsBytes) g = 1;
        }
        const int64_t items = g ? p.N * ((d.P + g - 1) / g) * ((full + cw - 1) / cw) : 0;
        if (g && items <= lim) {
            d.band_items = items;
            d.band_g = int32_t(g);
            d.band_cw = int32_t(cw);
            d.band_br = int32_t(br_of(g));
            d.band_tw = int32_t(nhwc ? p.W * p.C : tw_of(cw));
            d.band_wl = int32_t(wl_of(cw));
            d.band_cs = int32_t(cs_of(g, cw));
            d.band_lds = int32_t(lds_of(g, cw));
        }
    }
    return CONV_OK;
}

// Names of the contraction kernels for forced choices, with their variant
// counts (the candidates conv_tune times).
struct KernelFamily {
    const char* name;
    int kernel;
    int variants;
};
constexpr KernelFamily kKernelFamilies[] = {
    {"reg", KERN_REG, count_of(kRegVariants)},
    {"dma", KERN_DMA, count_of(kDmaVariants)},
    {"wide", KERN_WIDE, count_of(kWideVariants)},
    {"nchw", KERN_NCHW, count_of(kNchwVariants)},
    {"strip", KERN_STRIP, count_of(kStripVariants)},
    {"striprb", KERN_STRIP_RB, count_of(kStripRbVariants)},
    {"nchwstrip", KERN_NCHW_STRIP, count_of(kNchwStripVariants)},
    {"nchwtile", KERN_NCHW_TILE, count_of(kNchwTileVariants)},
    {"tile16", KERN_TILE16, count_of(kTile16Variants)},
    {"streamk", KERN_STREAMK, count_of(kDmaVariants)},
    {"striprb2", KERN_STRIP_RB2, count_of(kStripRb2Variants)},
    {"nchwtaps", KERN_NCHW_TAPS, count_of(kNchwTapsVariants)},
    {"striprb3", KERN_STRIP_RB3, count_of(kStripRb3Variants)},
    {"striprb4", KERN_STRIP_RB4, count_of(kStripRb4Variants)},
    {"stream1x1", KERN_STREAM1X1, count_of(kStream1x1Variants)},
};

// A ConvLSTM step: the gate convolution over concat(x, h) of p (C = c_x +
// hidden channels, K = 4 * hidden, stride 1, output the size of the input),
// fp32 NCHW, lowered (im2win or im2col) so that the lowering reads the two
// tensors; hidden channels a multiple of 16 (64 packed gate rows per tile).
conv_status_t plan_lstm(const conv_params_t& p, int64_t c_x, conv_desc& d) {
    if (p.layout != CONV_NCHW || p.dtype != CONV_F32) return CONV_ERR_UNSUPPORTED;
    if (p.algo != CONV_ALGO_IM2WIN && p.algo != CONV_ALGO_IM2COL) return CONV_ERR_UNSUPPORTED;
    if (c_x <= 0 || p.K <= 0 || p.K % 4 != 0 || p.C != c_x + p.K / 4) return CONV_ERR_INVALID_ARG;
    if (p.stride_h != 1 || p.stride_w != 1) return CONV_ERR_INVALID_ARG;
    if ((p.K / 4) % 16 != 0) return CONV_ERR_UNSUPPORTED;
    conv_status_t s = plan(p, d, nullptr, true);
    if (s != CONV_OK) return s;
    if (d.P != p.H || d.Q != p.W) return CONV_ERR_INVALID_ARG;
    if (d.bytes_low / 16 > 0xffffffffull) return CONV_ERR_UNSUPPORTED;
    d.lstm_cx = c_x;
    d.kernel = KERN_DMA;
    d.variant = -1;   // the dedicated ConvLSTM tile (kLstmVariant): no split contraction
    if (d.ksplit > 1) {
        d.ws_bytes = d.off_part;
        d.off_part = d.bytes_part = 0;
    }
    d.ksplit = 1;
    d.tile_order = CONV_TILE_LINEAR;
    d.tile_m = kLstmVariant.bm;
    d.tile_n = kLstmVariant.bn;
    d.tile_k = kLstmVariant.bk / 2;
    return CONV_OK;
}

// ---------------------------------------------------------------- pointer checks

conv_status_t check_dev(const void* ptr, size_t align) {
    if (!ptr) return CONV_ERR_NULL_PTR;
    if (reinterpret_cast<uintptr_t>(ptr) % align) return CONV_ERR_MISALIGNED;
    hipPointerAttribute_t attr;
    hipError_t e = hipPointerGetAttributes(&attr, ptr);
    if (e != hipSuccess) {
        (void)hipGetLastError();   // clear the sticky error of the failed query
        return CONV_ERR_NOT_DEVICE_PTR;
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged && attr.type != hipMemoryTypeUnified)
        return CONV_ERR_NOT_DEVICE_PTR;
    return CONV_OK;
}

// NHWC band staging moves 16-byte vectors when every x row starts on one.
bool band_vload(const conv_desc& d, const void* x) {
    return d.band_items && d.p.layout == CONV_NHWC && (int64_t(d.p.W) * d.p.C * d.elem) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(x) % 16 == 0;
}

// NCHW band staging moves 16-byte vectors when one chunk spans every column
// and every channel plane of x (and of the second input) starts on one; its
// offsets within a plane are 32-bit.
bool band_vload_nchw(const conv_desc& d, const void* x, const void* x2) {
    const int64_t full = d.p.algo == CONV_ALGO_IM2WIN ? d.W_used : d.Q;
    const int64_t plane = int64_t(d.p.H) * d.p.W;
    return d.band_items && d.p.layout == CONV_NCHW && d.band_cw == full && (plane * d.elem) % 16 == 0 &&
           plane < (int64_t(1) << 31) - 64 && reinterpret_cast<uintptr_t>(x) % 16 == 0 &&
           reinterpret_cast<uintptr_t>(x2) % 16 == 0;
}

LowerArgs lower_args(const conv_desc& d, const void* x, void* out) {
    LowerArgs a;
    a.x = x;
    a.out = out;
    a.N = int32_t(d.p.N);
    a.C = int32_t(d.p.C);
    a.H = int32_t(d.p.H);
    a.W = int32_t(d.p.W);
    a.P = int32_t(d.P);
    a.Q = int32_t(d.Q);
    a.R = int32_t(d.p.R);
    a.S = int32_t(d.p.S);
    a.sh = d.p.stride_h;
    a.sw = d.p.stride_w;
    a.ph = d.p.pad_h;
    a.pw = d.p.pad_w;
    a.dh = d.p.dil_h;
    a.dw = d.p.dil_w;
    a.W_used = int32_t(d.W_used);
    a.RCp = int32_t(d.RCp);
    a.Kl = int32_t(d.Kl);
    a.x2 = nullptr;
    a.C1 = int32_t(d.p.C);
    // (divisors the chosen kernel does not use may exceed 32 bits: clamped, never zero)
    auto fd = [](int64_t v) { return make_fastdiv(uint32_t(std::min<int64_t>(std::max<int64_t>(v, 1), INT32_MAX))); };
    const bool win = d.p.algo == CONV_ALGO_IM2WIN;
    const int64_t vpc = (win ? d.RCp : d.Kl) / d.vec;
    const int64_t full = win ? d.W_used : d.Q;
    a.G = d.band_g;
    a.CW = d.band_items ? d.band_cw : int32_t(full);
    a.BR = d.band_br;
    a.WL = d.band_wl;
    a.CS = d.band_cs;
    a.TW = band_vload(d, x) ? d.band_tw / d.vec : d.band_tw;
    a.fd_cb = fd(d.band_items ? (full + d.band_cw - 1) / d.band_cw : 1);
    a.fd_pb = fd(d.band_items ? (d.P + d.band_g - 1) / d.band_g : 1);
    a.fd_tw = fd(a.TW);
    a.fd_br = fd(d.band_br);
    a.fd_row = fd(int64_t(a.CW) * vpc);
    a.fd_vpc = fd(vpc);
    a.fd_cpv = fd(d.RCp / d.vec);
    a.fd_c = fd(d.p.C);
    a.fd_p = fd(d.P);
    a.fd_q = fd(d.Q);
    a.fd_nv = fd((int64_t(d.band_br) * d.p.W + d.vec - 1) / d.vec + 1);
    a.fd_w = fd(d.p.W);
    if (d.unpadded) {
        // element decode: per strip (im2win) or per row (im2col), per window row
        a.fd_row = fd(win ? d.W_used * d.RCp : d.Kl);
        a.fd_cpv = fd(d.RCp);
    }
    return a;
}

uint32_t grid_stride_blocks(uint64_t work) {
    uint64_t b = (work + 255) / 256;
    const uint64_t cap = 256ull * 64;   // 64 blocks per CU is plenty for a streaming copy
    return uint32_t(b < cap ? (b ? b : 1) : cap);
}

// ---------------------------------------------------------------- launches

template <typename T>
void launch_pack(const conv_desc& d, const void* w, void* out, hipStream_t st) {
    if (d.kernel == KERN_TILE16) {
        if constexpr (sizeof(T) == 2) {
            const Tile16Variant& v = kTile16Variants[d.variant];
            Tile16PackArgs a{w, out, int32_t(d.p.K), int32_t(d.p.C), int32_t(d.p.R), int32_t(d.p.S), d.p.pad_w,
                             v.ks, v.tn, v.split};
            pack_filter_tile16_kernel<T><<<(v.ks * v.tn * v.split * 64 + 255) / 256, 256, 0, st>>>(a);
        }
        return;
    }
    if (d.frag_pack && (d.kernel == KERN_STRIP_RB3 || d.kernel == KERN_STRIP_RB4)) {
        if constexpr (sizeof(T) == 2) {
            const int32_t NB = int32_t((d.p.K + 15) / 16);
            FragPackArgs a{w, out, int32_t(d.p.K), int32_t(d.Kg), NB};
            pack_filter_frag16_kernel<T><<<grid_stride_blocks(uint64_t(NB) * (d.Kg / 32) * 64), 256, 0, st>>>(a);
        }
        return;
    }
    if (d.frag_pack) {
        if constexpr (sizeof(T) == 2) {
            const int32_t NB = int32_t((d.p.K + 31) / 32);
            FragPackArgs a{w, out, int32_t(d.p.K), int32_t(d.Kg), NB};
            pack_filter_frag_kernel<T><<<grid_stride_blocks(uint64_t(NB) * (d.Kg / 16) * 64), 256, 0, st>>>(a);
        } else {
            const int32_t NB = int32_t((d.p.K + 15) / 16);
            FragPackF32Args a{w, out, int32_t(d.p.K), int32_t(d.p.C), int32_t(d.p.R), int32_t(d.p.S), NB};
            pack_filter_frag_f32_kernel<<<grid_stride_blocks(uint64_t(NB) * (d.Kg / 16) * 64), 256, 0, st>>>(a);
        }
        return;
    }
    PackArgs a{w,
               out,
               int32_t(d.p.K),
               int32_t(d.p.C),
               int32_t(d.p.R),
               int32_t(d.p.S),
               int32_t(d.RCp),
               int32_t(d.Kl),
               int32_t(d.lstm_cx ? d.p.K / 4 : 0)};
    const uint32_t blocks = grid_stride_blocks(uint64_t(d.p.K) * d.Kl);
    if (d.p.layout == CONV_NHWC)
        pack_filter_kernel<T, true><<<blocks, 256, 0, st>>>(a);
    else
        pack_filter_kernel<T, false><<<blocks, 256, 0, st>>>(a);
}

// Band lowering of one item per block (band_items > 0).
template <typename T>
void launch_band(const conv_desc& d, const LowerArgs& a, bool vload, hipStream_t st) {
    const bool col = d.p.algo != CONV_ALGO_IM2WIN;
    const dim3 grid(uint32_t(d.band_items));
    const size_t lds = size_t(d.band_lds);
    if (d.p.layout == CONV_NCHW) {
        const bool v = band_vload_nchw(d, a.x, a.x2);
        if (col && v)
            lower_nchw_band_kernel<T, true, true><<<grid, 256, lds, st>>>(a);
        else if (col)
            lower_nchw_band_kernel<T, true, false><<<grid, 256, lds, st>>>(a);
        else if (v)
            lower_nchw_band_kernel<T, false, true><<<grid, 256, lds, st>>>(a);
        else
            lower_nchw_band_kernel<T, false, false><<<grid, 256, lds, st>>>(a);
    } else if (vload) {
        if (col)
            lower_nhwc_band_kernel<T, true, true><<<grid, 256, lds, st>>>(a);
        else
            lower_nhwc_band_kernel<T, false, true><<<grid, 256, lds, st>>>(a);
    } else {
        if (col)
            lower_nhwc_band_kernel<T, true, false><<<grid, 256, lds, st>>>(a);
        else
            lower_nhwc_band_kernel<T, false, false><<<grid, 256, lds, st>>>(a);
    }
}

template <typename T>
void launch_lower_args(const conv_desc& d, const LowerArgs& a, hipStream_t st) {
    constexpr int VEC = Vec<T>::n;
    const bool nhwc = d.p.layout == CONV_NHWC;
    const bool win = d.p.algo == CONV_ALGO_IM2WIN;
    const uint64_t total = (win ? d.im2win_bytes : uint64_t(d.M) * d.Kl * d.elem) / 16;
    if (d.unpadded) {
        const uint64_t elems = win ? d.im2win_bytes / d.elem : uint64_t(d.M) * d.Kl;
        const uint32_t nv = uint32_t((elems + VEC - 1) / VEC);
        if (nhwc && win)
            lower_unpadded_kernel<T, true, false><<<grid_stride_blocks(nv), 256, 0, st>>>(a, nv, uint32_t(elems));
        else if (nhwc)
            lower_unpadded_kernel<T, true, true><<<grid_stride_blocks(nv), 256, 0, st>>>(a, nv, uint32_t(elems));
        else if (win)
            lower_unpadded_kernel<T, false, false><<<grid_stride_blocks(nv), 256, 0, st>>>(a, nv, uint32_t(elems));
        else
            lower_unpadded_kernel<T, false, true><<<grid_stride_blocks(nv), 256, 0, st>>>(a, nv, uint32_t(elems));
    } else if (nhwc && d.p.C % VEC == 0) {
        if (win) {
            const uint32_t vps = uint32_t(d.W_used * d.RCp / VEC);
            dim3 grid(uint32_t(d.p.N * d.P), (vps + 256 * LOWER_U - 1) / (256 * LOWER_U));
            im2win_nhwc_vec_kernel<T><<<grid, 256, 0, st>>>(a);
        } else {
            const uint32_t blocks = grid_stride_blocks((total + LOWER_U - 1) / LOWER_U);
            im2col_nhwc_vec_kernel<T><<<blocks, 256, 0, st>>>(a, uint32_t(total));
        }
    } else if (d.band_items > 0) {
        launch_band<T>(d, a, band_vload(d, a.x), st);
    } else if (nhwc) {
        if (win)
            lower_generic_kernel<T, true, false><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
        else
            lower_generic_kernel<T, true, true><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
    } else {
        if (win)
            lower_generic_kernel<T, false, false><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
        else
            lower_generic_kernel<T, false, true><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
    }
}

template <typename T>
void launch_lower(const conv_desc& d, const void* x, void* out, hipStream_t st) {
    launch_lower_args<T>(d, lower_args(d, x, out), st);
}

template <template <typename> class F, typename... Args>
void by_dtype(conv_dtype_t dt, Args&&... args) {
    switch (dt) {
        case CONV_F32: F<float>::run(args...); break;
        case CONV_F16: F<_Float16>::run(args...); break;
        default: F<__bf16>::run(args...); break;
    }
}

template <typename T>
struct PackOp {
    static void run(const conv_desc& d, const void* w, void* out, hipStream_t st) { launch_pack<T>(d, w, out, st); }
};
template <typename T>
struct LowerOp {
    static void run(const conv_desc& d, const void* x, void* out, hipStream_t st) { launch_lower<T>(d, x, out, st); }
};
template <typename T>
struct GemmOp {
    static void run(const conv_desc& d, const void* x, const void* w, const void* bias, void* y, const void* ws,
                    uint32_t epoch, hipStream_t st) {
        launch_gemm<T>(d, x, w, bias, y, ws, epoch, st);
    }
};

// Launch epochs (stream-K flags): one counter for the process, so that no
// two launches sharing a workspace use the same value; 0 is never used.
std::atomic<uint32_t> g_epoch{0};
uint32_t next_epoch() {
    uint32_t e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    while (e == 0) e = g_epoch.fetch_add(1, std::memory_order_relaxed) + 1;
    return e;
}

conv_status_t launch_status() { return from_hip(hipGetLastError()); }

conv_status_t check_ws(const conv_desc& d, const void* ws) {
    if (d.ws_bytes == 0) return CONV_OK;
    return check_dev(ws, 16);
}

// Unchecked stage launches (pointers already validated by the caller).
conv_status_t run_pack(const conv_desc& d, const void* w, void* ws, hipStream_t st) {
    if (!(d.pack || d.frag_pack) || d.p.N == 0) return CONV_OK;
    by_dtype<PackOp>(d.p.dtype, d, w, static_cast<char*>(ws) + d.off_filter, st);
    return launch_status();
}

conv_status_t run_lower(const conv_desc& d, const void* x, void* ws, hipStream_t st) {
    if (d.elided || d.p.N == 0) return CONV_OK;
    by_dtype<LowerOp>(d.p.dtype, d, x, static_cast<char*>(ws) + d.off_low, st);
    return launch_status();
}

conv_status_t run_contract(const conv_desc& d, const void* x, const void* w, const void* bias, void* y,
                           const void* ws, hipStream_t st) {
    if (d.p.N == 0) return CONV_OK;
    by_dtype<GemmOp>(d.p.dtype, d, x, w, bias, y, ws, next_epoch(), st);
    return launch_status();
}

// ConvLSTM step: lowering of concat(x, h_prev), then the gate contraction
// with the cell update.
conv_status_t run_lstm(const conv_desc& d, const void* x, const void* h_prev, const void* c_prev, const void* bias,
                       void* h_out, void* c_out, void* ws, hipStream_t st) {
    if (d.p.N == 0) return CONV_OK;
    LowerArgs a = lower_args(d, x, static_cast<char*>(ws) + d.off_low);
    a.x2 = h_prev;
    a.C1 = int32_t(d.lstm_cx);
    launch_lower_args<float>(d, a, st);
    conv_status_t s = launch_status();
    if (s != CONV_OK) return s;
    launch_lstm_gemm(d, bias, c_prev, h_out, c_out, ws, st);
    return launch_status();
}

// ---------------------------------------------------------------- scratch of conv2d_fwd_noalloc

// The workspace of conv2d_fwd_noalloc: a fixed array in device memory (each
// GPU the library runs on holds its own copy until the process ends).  Its
// name is a host-side stand-in, never a device address: host code only ever
// uses the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[CONV_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch[kScratchDevices];

// This device's copy of `scratch`, looked up once per device with that
// device current (the first call on it) and kept.
conv_status_t scratch_ptr(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return CONV_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return CONV_ERR_UNSUPPORTED;
    void* p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return CONV_ERR_HIP;
        }
        g_scratch[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return CONV_OK;
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

conv_status_t conv_create_desc_forced(const conv_params_t* p, const char* force, conv_desc_t* out) {
    if (!p || !out) return CONV_ERR_NULL_PTR;
    *out = nullptr;
    conv_desc tmp{};
    tmp.p = *p;
    conv_status_t s = plan(*p, tmp, force);
    if (s != CONV_OK) return s;
    conv_desc* d = new (std::nothrow) conv_desc(tmp);
    if (!d) return CONV_ERR_OOM;
    d->magic = kDescMagic;
    *out = d;
    return CONV_OK;
}

conv_status_t conv_create_desc(const conv_params_t* p, conv_desc_t* out) {
    return conv_create_desc_forced(p, nullptr, out);
}

conv_status_t conv_lstm_create_desc(const conv_params_t* p, int64_t c_x, conv_desc_t* out) {
    if (!p || !out) return CONV_ERR_NULL_PTR;
    *out = nullptr;
    conv_desc tmp{};
    tmp.p = *p;
    conv_status_t s = plan_lstm(*p, c_x, tmp);
    if (s != CONV_OK) return s;
    conv_desc* d = new (std::nothrow) conv_desc(tmp);
    if (!d) return CONV_ERR_OOM;
    d->magic = kDescMagic;
    *out = d;
    return CONV_OK;
}

conv_status_t conv_lstm_step(conv_desc_t d, const void* x, const void* h_prev, const void* c_prev, const void* w,
                             const void* bias, void* h_out, void* c_out, void* ws, void* stream) {
    if (!desc_ok(d) || d->lstm_cx == 0) return CONV_ERR_INVALID_ARG;
    if (d->p.N == 0) return CONV_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    conv_status_t s;
    for (const void* ptr : {x, h_prev, c_prev, w, static_cast<const void*>(h_out), static_cast<const void*>(c_out)})
        if ((s = check_dev(ptr, 16)) != CONV_OK) return s;
    if (bias && (s = check_dev(bias, 4)) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    if ((s = run_pack(*d, w, ws, st)) != CONV_OK) return s;
    return run_lstm(*d, x, h_prev, c_prev, bias, h_out, c_out, ws, st);
}

conv_status_t conv_destroy_desc(conv_desc_t d) {
    if (!d) return CONV_OK;
    if (d->magic != kDescMagic) return CONV_ERR_INVALID_ARG;
    d->magic = 0;
    delete d;
    return CONV_OK;
}

conv_status_t conv_workspace_size(conv_desc_t d, size_t* bytes) {
    if (!bytes) return CONV_ERR_NULL_PTR;
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
    *bytes = size_t(d->ws_bytes);
    return CONV_OK;
}

conv_status_t conv_output_dims(conv_desc_t d, int64_t* P, int64_t* Q) {
    if (!P || !Q) return CONV_ERR_NULL_PTR;
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
    *P = d->P;
    *Q = d->Q;
    return CONV_OK;
}

conv_status_t conv_plan_info(conv_desc_t d, conv_plan_info_t* info) {
    if (!info) return CONV_ERR_NULL_PTR;
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
    conv_plan_info_t i{};
    i.P = d->P;
    i.Q = d->Q;
    i.M = d->M;
    i.Kg = d->Kg;
    i.W_used = d->W_used;
    i.RCp = d->RCp;
    i.Kl = d->Kl;
    i.ws_bytes = d->ws_bytes;
    i.ws_filter_offset = d->off_filter;
    i.ws_filter_bytes = d->bytes_filter;
    i.ws_lowered_offset = d->off_low;
    i.ws_lowered_bytes = d->bytes_low;
    i.im2win_bytes = d->im2win_bytes;
    i.im2col_bytes = d->im2col_bytes;
    i.lowering_elided = d->elided ? 1 : 0;
    i.tile_m = d->tile_m;
    i.tile_n = d->tile_n;
    i.tile_k = d->tile_k;
    i.elem_bytes = d->elem;
    i.kernel = d->kernel;
    i.kernel_variant = d->variant;
    i.ws_partial_offset = d->off_part;
    i.ws_partial_bytes = d->bytes_part;
    i.ksplit = d->ksplit;
    i.tile_order = d->tile_order;
    *info = i;
    return CONV_OK;
}

conv_status_t conv_pack_filter(conv_desc_t d, const void* w, void* ws, void* stream) {
    if (!desc_ok(d) || d->lstm_cx) return CONV_ERR_INVALID_ARG;
    if (!(d->pack || d->frag_pack) || d->p.N == 0) return CONV_OK;
    conv_status_t s;
    if ((s = check_dev(w, 16)) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    return run_pack(*d, w, ws, static_cast<hipStream_t>(stream));
}

conv_status_t conv_lower_input(conv_desc_t d, const void* x, void* ws, void* stream) {
    if (!desc_ok(d) || d->lstm_cx) return CONV_ERR_INVALID_ARG;
    if (d->elided || d->p.N == 0) return CONV_OK;
    conv_status_t s;
    if ((s = check_dev(x, 16)) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    return run_lower(*d, x, ws, static_cast<hipStream_t>(stream));
}

conv_status_t conv_contract(conv_desc_t d, const void* x, const void* w, const void* bias, void* y, void* ws,
                            void* stream) {
    if (!desc_ok(d) || d->lstm_cx) return CONV_ERR_INVALID_ARG;
    if (d->p.N == 0) return CONV_OK;
    conv_status_t s;
    if ((s = check_dev(y, 16)) != CONV_OK) return s;
    if (d->elided && (s = check_dev(x, 16)) != CONV_OK) return s;
    if (!d->pack && (s = check_dev(w, 16)) != CONV_OK) return s;
    if (bias && (s = check_dev(bias, size_t(d->elem))) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    return run_contract(*d, x, w, bias, y, ws, static_cast<hipStream_t>(stream));
}

conv_status_t conv2d_fwd(conv_desc_t d, const void* x, const void* w, const void* bias, void* y, void* ws,
                         void* stream) {
    if (!desc_ok(d) || d->lstm_cx) return CONV_ERR_INVALID_ARG;
    if (d->p.N == 0) return CONV_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    conv_status_t s;
    // Validate every pointer before anything is enqueued.
    if ((s = check_dev(x, 16)) != CONV_OK) return s;
    if ((s = check_dev(w, 16)) != CONV_OK) return s;
    if ((s = check_dev(y, 16)) != CONV_OK) return s;
    if (bias && (s = check_dev(bias, size_t(d->elem))) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    if ((s = run_pack(*d, w, ws, st)) != CONV_OK) return s;
    if ((s = run_lower(*d, x, ws, st)) != CONV_OK) return s;
    return run_contract(*d, x, w, bias, y, ws, st);
}

conv_status_t conv2d_fwd_noalloc(conv_desc_t d, const void* x, const void* w, const void* bias, void* y,
                                 void* stream) {
    if (!desc_ok(d) || d->lstm_cx) return CONV_ERR_INVALID_ARG;
    if (d->ws_bytes > CONV_NOALLOC_SCRATCH_BYTES) return CONV_ERR_UNSUPPORTED;
    if (d->p.N == 0) return CONV_OK;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    conv_status_t s;
    if ((s = check_dev(x, 16)) != CONV_OK) return s;
    if ((s = check_dev(w, 16)) != CONV_OK) return s;
    if ((s = check_dev(y, 16)) != CONV_OK) return s;
    if (bias && (s = check_dev(bias, size_t(d->elem))) != CONV_OK) return s;
    // Every kernel writes each workspace byte it reads before reading it
    // (packed filters, lowered rows, split partial sums), so the scratch left
    // by an earlier call needs no clearing.
    void* ws = nullptr;
    if (d->ws_bytes && (s = scratch_ptr(&ws)) != CONV_OK) return s;
    if ((s = run_pack(*d, w, ws, st)) != CONV_OK) return s;
    if ((s = run_lower(*d, x, ws, st)) != CONV_OK) return s;
    return run_contract(*d, x, w, bias, y, ws, st);
}

conv_status_t conv_tune(conv_desc_t d, const void* x, const void* w, const void* bias, void* y, void* ws,
                        size_t ws_bytes, int32_t reps, void* stream, conv_desc_t* tuned,
                        conv_tune_result_t* result) {
    if (!tuned || !result) return CONV_ERR_NULL_PTR;
    *tuned = nullptr;
    if (!desc_ok(d) || d->lstm_cx || reps < 1) return CONV_ERR_INVALID_ARG;
    *result = conv_tune_result_t{};
    result->kernel = d->kernel;
    result->kernel_variant = d->variant;
    result->ksplit = d->ksplit;
    result->tile_order = d->tile_order;
    // the kept plan goes into a new descriptor; d stays as it is
    auto emit = [&](const conv_desc& c) -> conv_status_t {
        conv_desc* nd = new (std::nothrow) conv_desc(c);
        if (!nd) return CONV_ERR_OOM;
        nd->magic = kDescMagic;
        *tuned = nd;
        return CONV_OK;
    };
    if (d->p.N == 0) return emit(*d);
    const hipStream_t st = static_cast<hipStream_t>(stream);
    conv_status_t s;
    if ((s = check_dev(x, 16)) != CONV_OK) return s;
    if ((s = check_dev(w, 16)) != CONV_OK) return s;
    if ((s = check_dev(y, 16)) != CONV_OK) return s;
    if (bias && (s = check_dev(bias, size_t(d->elem))) != CONV_OK) return s;
    if (ws_bytes < d->ws_bytes) return CONV_ERR_INVALID_ARG;
    if (ws_bytes && (s = check_dev(ws, 16)) != CONV_OK) return s;

    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess) return CONV_ERR_HIP;
    if (hipEventCreate(&e1) != hipSuccess) {
        (void)hipEventDestroy(e0);
        return CONV_ERR_HIP;
    }
    // ms per call of one plan: one untimed call, then reps timed ones.
    auto time_plan = [&](const conv_desc& c, float* ms) -> conv_status_t {
        conv_status_t r;
        for (int i = 0; i <= reps; ++i) {
            if (i == 1 && hipEventRecord(e0, st) != hipSuccess) return CONV_ERR_HIP;
            if ((r = run_pack(c, w, ws, st)) != CONV_OK) return r;
            if ((r = run_lower(c, x, ws, st)) != CONV_OK) return r;
            if ((r = run_contract(c, x, w, bias, y, ws, st)) != CONV_OK) return r;
        }
        if (hipEventRecord(e1, st) != hipSuccess || hipEventSynchronize(e1) != hipSuccess) return CONV_ERR_HIP;
        float t = 0.f;
        if (hipEventElapsedTime(&t, e0, e1) != hipSuccess) return CONV_ERR_HIP;
        *ms = t / float(reps);
        return CONV_OK;
    };
    conv_desc best = *d;
    float best_ms = 0.f;
    s = time_plan(*d, &best_ms);
    result->default_ms = best_ms;
    int n = 1;
    for (const KernelFamily& f : kKernelFamilies) {
        // the pipelined and wide-tile kernels also without and with a split
        // contraction (2, 4)
        const bool splits = f.kernel == KERN_DMA || f.kernel == KERN_WIDE;
        const int nks = splits ? 3 : 1;
        for (int v = 0; v < f.variants && s == CONV_OK; ++v) {
            for (int si = 0; si < nks && s == CONV_OK; ++si) {
                char force[32];
                if (splits)
                    std::snprintf(force, sizeof(force), "%s:%d:%d", f.name, v, 1 << si);
                else
                    std::snprintf(force, sizeof(force), "%s:%d", f.name, v);
                conv_desc c{};
                c.p = d->p;
                if (plan(d->p, c, force) != CONV_OK || c.kernel != f.kernel || c.variant != v) continue;
                if (splits && c.ksplit != (1 << si)) continue;   // clamped: same as another candidate
                if (c.ws_bytes > ws_bytes ||
                    (c.kernel == d->kernel && c.variant == d->variant && c.ksplit == d->ksplit))
                    continue;
                float ms = 0.f;
                s = time_plan(c, &ms);
                ++n;
                if (s == CONV_OK && ms < best_ms) {
                    best = c;
                    best_ms = ms;
                }
            }
        }
    }
    // the pipelined kernel's tile orders, on the fastest plan
    if (best.kernel == KERN_DMA) {
        const conv_desc base = best;
        for (int o = CONV_TILE_LINEAR; o <= CONV_TILE_XCD_COLS && s == CONV_OK; ++o) {
            if (o == base.tile_order) continue;
            conv_desc c = base;
            c.tile_order = o;
            float ms = 0.f;
            s = time_plan(c, &ms);
            ++n;
            if (s == CONV_OK && ms < best_ms) {
                best = c;
                best_ms = ms;
            }
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (s != CONV_OK) return s;
    if ((s = emit(best)) != CONV_OK) return s;
    result->candidates = n;
    result->kernel = best.kernel;
    result->kernel_variant = best.variant;
    result->ksplit = best.ksplit;
    result->tile_order = best.tile_order;
    result->best_ms = best_ms;
    return CONV_OK;
}

const char* conv_status_string(conv_status_t s) {
    switch (s) {
        case CONV_OK: return "success";
        case CONV_ERR_INVALID_ARG: return "invalid argument";
        case CONV_ERR_UNSUPPORTED: return "unsupported convolution";
        case CONV_ERR_NULL_PTR: return "null pointer";
        case CONV_ERR_NOT_DEVICE_PTR: return "pointer is not device memory";
        case CONV_ERR_MISALIGNED: return "pointer misaligned";
        case CONV_ERR_HIP: return "HIP runtime error";
        case CONV_ERR_OOM: return "out of host memory";
    }
    return "unknown status";
}

}  // extern "C"
