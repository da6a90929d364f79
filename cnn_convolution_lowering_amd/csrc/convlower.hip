// C ABI of the convolution library: descriptor (plan), validation, and the
// launches of the filter pack, the lowering (im2win / im2col) and the MFMA
// contraction.  Every declaration is in include/convlower.h.
//
// The descriptor is pure host arithmetic (no HIP call), so shapes, workspace
// sizes and error codes can be checked without a GPU.  The launch entry
// points make no allocation and no synchronisation: they validate pointers,
// enqueue kernels on the caller's stream and report launch errors.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <new>

#include "../../include/convlower.h"
#include "igemm.hpp"
#include "igemm_dma.hpp"
#include "igemm_nchw.hpp"
#include "lowering.hpp"

using namespace convlower;

namespace {

constexpr uint32_t kDescMagic = 0x636f6e76u;   // marks a live descriptor
constexpr uint64_t kWsAlign = 256;             // workspace sub-buffer alignment (bytes)
constexpr int kStageLdsBytes = 32 * 1024;      // NCHW staging tile budget per block

enum TileId : int32_t {
    TILE_128x128 = 0,
    TILE_128x64 = 1,
    TILE_128x32 = 2,
    TILE_256x128 = 3,   // pipelined (LDS-DMA) kernel only
    TILE_64x128 = 4,    // fp32 NCHW pipelined kernel only
};

}  // namespace

// Variants of the fp32 NCHW fused kernel (BM, BN, BK, STAGES).  The default
// per shape (see plan) follows a sweep of all of them on the encoder layers;
// CONVLOWER_NCHW_VARIANT=<index> forces one, for tuning.
struct NchwVariant {
    int bm, bn, bk, stages;
};
constexpr NchwVariant kNchwVariants[] = {
    {128, 32, 32, 3}, {128, 64, 32, 3}, {128, 128, 32, 3}, {64, 128, 32, 3},
    {128, 64, 16, 4}, {128, 64, 16, 6}, {64, 64, 32, 4},  {64, 64, 16, 6},
    {128, 32, 16, 4},
};
constexpr int kNchwVariantCount = sizeof(kNchwVariants) / sizeof(kNchwVariants[0]);

struct conv_desc {
    uint32_t magic;
    conv_params_t p;
    int64_t P, Q, M, Kg, W_used, RCp, Kl;
    int32_t elem, vec;
    bool elided;        // no lowering launch: the contraction reads x (implicit, or 1x1 NHWC unpadded)
    bool pack;          // filter needs packing into ws
    uint64_t off_filter, bytes_filter, off_low, bytes_low, ws_bytes;
    uint64_t im2win_bytes, im2col_bytes;
    int32_t tile;       // TileId
    bool dma;           // pipelined LDS-DMA contraction kernel
    bool nchw_dma;      // pipelined fp32 NCHW fused kernel
    int32_t nchw_variant;   // index into kNchwVariants
    int32_t tile_m, tile_n, tile_k;
    // NCHW staging (0 = use the element-wise kernel)
    int32_t stage_chunk, stage_ld;
};

namespace {

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

bool desc_ok(conv_desc_t d) { return d != nullptr && d->magic == kDescMagic; }

conv_status_t from_hip(hipError_t e) { return e == hipSuccess ? CONV_OK : CONV_ERR_HIP; }

// ---------------------------------------------------------------- planning

conv_status_t plan(const conv_params_t& p, conv_desc& d) {
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
    d.RCp = int64_t(round_up(uint64_t(p.R * p.C), uint64_t(d.vec)));
    d.Kl = p.S * d.RCp;
    d.W_used = (d.Q - 1) * p.stride_w + (p.S - 1) * int64_t(p.dil_w) + 1;

    const bool nhwc = p.layout == CONV_NHWC;
    const bool c_vec = p.C % d.vec == 0;
    const bool implicit = p.algo == CONV_ALGO_IMPLICIT;
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
    if (!d.elided && low_vec > 0xffffffffull) return CONV_ERR_UNSUPPORTED;
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
    const bool a_chunks = implicit ? (nhwc && c_vec) : true;
    d.dma = a_chunks && a_bytes < (uint64_t(1) << 31) && b_bytes < (uint64_t(1) << 31);
    // Tile: BN covers the output channels up to 128; BM = 256 where that still
    // gives two workgroups per CU, else 128.
    d.tile = p.K <= 32 ? TILE_128x32 : (p.K <= 64 ? TILE_128x64 : TILE_128x128);
    if (d.dma && d.tile == TILE_128x128 && (d.M / 256) * ((p.K + 127) / 128) >= 512) d.tile = TILE_256x128;
    // fp32 NCHW fused windows: the pipelined kernel with 4-byte window loads.
    d.nchw_dma = implicit && !nhwc && p.dtype == CONV_F32 && x_bytes < (uint64_t(1) << 31) &&
                 b_bytes < (uint64_t(1) << 31);
    if (d.nchw_dma && d.tile == TILE_128x128 && (d.M / 128) * ((p.K + 127) / 128) < 512) d.tile = TILE_64x128;
    d.tile_m = d.tile == TILE_256x128 ? 256 : (d.tile == TILE_64x128 ? 64 : 128);
    d.tile_n = d.tile == TILE_128x32 ? 32 : (d.tile == TILE_128x64 ? 64 : 128);
    d.tile_k = p.dtype == CONV_F32 ? 16 : 32;
    // fp32 NCHW: narrow K -> 128-row tiles, 16-deep stages x4; wide K -> 64-row
    // tiles, 64 or 128 channels wide depending on how many workgroups that gives.
    if (p.K <= 32)
        d.nchw_variant = 8;
    else if (p.K <= 64)
        d.nchw_variant = 4;
    else
        d.nchw_variant = (d.M / 64) * ((p.K + 127) / 128) >= 768 ? 3 : 7;
    if (d.nchw_dma) {
        // Tuning override: CONVLOWER_NCHW_VARIANT=<index> selects another compiled variant.
        if (const char* v = std::getenv("CONVLOWER_NCHW_VARIANT")) {
            const int i = std::atoi(v);
            if (i >= 0 && i < kNchwVariantCount) d.nchw_variant = i;
        }
        d.tile_m = kNchwVariants[d.nchw_variant].bm;
        d.tile_n = kNchwVariants[d.nchw_variant].bn;
        d.tile_k = kNchwVariants[d.nchw_variant].bk;
    }

    // NCHW staging tile: whole strip columns of R*C values per LDS row.
    d.stage_chunk = 0;
    d.stage_ld = 0;
    if (!nhwc) {
        const int64_t ld = p.R * p.C + 1;     // odd pitch spreads the column-major writes over banks
        const int64_t cols_fit = kStageLdsBytes / (ld * d.elem);
        if (p.algo == CONV_ALGO_IM2WIN) {
            if (cols_fit >= 1) {
                d.stage_chunk = int32_t(cols_fit < d.W_used ? cols_fit : d.W_used);
                d.stage_ld = int32_t(ld);
            }
        } else {
            // output columns per block: (chunk-1)*sw + (S-1)*dw + 1 strip columns must fit
            const int64_t span = (p.S - 1) * int64_t(p.dil_w) + 1;
            if (cols_fit >= span) {
                int64_t qc = (cols_fit - span) / p.stride_w + 1;
                if (qc > d.Q) qc = d.Q;
                d.stage_chunk = int32_t(qc);
                d.stage_ld = int32_t(ld);
            }
        }
    }
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
    a.chunk = d.stage_chunk;
    a.lds_ld = d.stage_ld;
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
    PackArgs a{w, out, int32_t(d.p.K), int32_t(d.p.C), int32_t(d.p.R), int32_t(d.p.S), int32_t(d.RCp), int32_t(d.Kl)};
    const uint32_t blocks = grid_stride_blocks(uint64_t(d.p.K) * d.Kl);
    if (d.p.layout == CONV_NHWC)
        pack_filter_kernel<T, true><<<blocks, 256, 0, st>>>(a);
    else
        pack_filter_kernel<T, false><<<blocks, 256, 0, st>>>(a);
}

template <typename T>
void launch_lower(const conv_desc& d, const void* x, void* out, hipStream_t st) {
    constexpr int VEC = Vec<T>::n;
    const LowerArgs a = lower_args(d, x, out);
    const bool nhwc = d.p.layout == CONV_NHWC;
    const bool c_vec = d.p.C % VEC == 0;
    if (d.p.algo == CONV_ALGO_IM2WIN) {
        if (nhwc) {
            const uint32_t vps = uint32_t(d.W_used * d.RCp / VEC);
            dim3 grid(uint32_t(d.p.N * d.P), (vps + 255) / 256);
            if (c_vec)
                im2win_nhwc_kernel<T, true><<<grid, 256, 0, st>>>(a);
            else
                im2win_nhwc_kernel<T, false><<<grid, 256, 0, st>>>(a);
        } else if (d.stage_chunk > 0) {
            dim3 grid(uint32_t(d.p.N * d.P), uint32_t((d.W_used + d.stage_chunk - 1) / d.stage_chunk));
            const size_t lds = size_t(d.stage_chunk) * d.stage_ld * sizeof(T);
            im2win_nchw_kernel<T><<<grid, 256, lds, st>>>(a);
        } else {
            const uint64_t total = d.im2win_bytes / 16;
            lower_generic_kernel<T, false, false><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
        }
    } else {
        const uint64_t total = uint64_t(d.M) * d.Kl / VEC;
        if (nhwc) {
            if (c_vec)
                im2col_nhwc_kernel<T, true><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
            else
                im2col_nhwc_kernel<T, false><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
        } else if (d.stage_chunk > 0) {
            dim3 grid(uint32_t(d.p.N * d.P), uint32_t((d.Q + d.stage_chunk - 1) / d.stage_chunk));
            const int64_t cols = int64_t(d.stage_chunk - 1) * d.p.stride_w + (d.p.S - 1) * int64_t(d.p.dil_w) + 1;
            const size_t lds = size_t(cols) * d.stage_ld * sizeof(T);
            im2col_nchw_kernel<T><<<grid, 256, lds, st>>>(a);
        } else {
            lower_generic_kernel<T, false, true><<<grid_stride_blocks(total), 256, 0, st>>>(a, uint32_t(total));
        }
    }
}

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

template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES, bool NHWC_OUT, class ASrc, class BSrc>
void launch_dma_core(const conv_desc& d, GemmArgs g, hipStream_t st) {
    g.tiles_n = int32_t((d.p.K + BN - 1) / BN);
    const uint64_t tiles_m = (uint64_t(d.M) + BM - 1) / BM;
    const uint32_t blocks = uint32_t(tiles_m * g.tiles_n);
    conv_gemm_dma_kernel<T, BM, BN, BK, WGM, WGN, STAGES, NHWC_OUT, ASrc, BSrc><<<blocks, 256, 0, st>>>(g);
}

template <typename T, int BM, int BN, int BK, int WGM, int WGN, int STAGES>
void launch_dma_tile(const conv_desc& d, const GemmArgs& g, hipStream_t st) {
    using B = DmaRows<T, BN, BK, false, false>;
    const bool nhwc = d.p.layout == CONV_NHWC;
    if (d.p.algo == CONV_ALGO_IMPLICIT) {
        // NHWC with C a whole number of vectors (checked when planning)
        if (d.p.C % BK == 0)
            launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, true, DmaWindowNHWCBlocked<T, BM, BK>, B>(d, g, st);
        else
            launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, true, DmaWindowNHWC<T, BM, BK>, B>(d, g, st);
    } else if (!d.elided && d.p.algo == CONV_ALGO_IM2WIN) {
        using A = DmaRows<T, BM, BK, true, true>;
        if (nhwc) launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, true, A, B>(d, g, st);
        else launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, A, B>(d, g, st);
    } else {
        using A = DmaRows<T, BM, BK, true, false>;
        if (nhwc) launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, true, A, B>(d, g, st);
        else launch_dma_core<T, BM, BN, BK, WGM, WGN, STAGES, false, A, B>(d, g, st);
    }
}

template <typename T>
void launch_gemm(const conv_desc& d, const void* x, const void* w, const void* bias, void* y, const void* ws,
                 hipStream_t st) {
    constexpr int BK = sizeof(T) == 4 ? 16 : 32;
    const char* wsb = static_cast<const char*>(ws);
    GemmArgs g{};
    g.b = d.pack ? static_cast<const void*>(wsb + d.off_filter) : w;
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
    if (d.nchw_dma) {
        if constexpr (sizeof(T) == 4) {
            auto launch = [&](auto kernel, int BM, int BN) {
                GemmArgs h = g;
                h.tiles_n = int32_t((d.p.K + BN - 1) / BN);
                const uint32_t blocks = uint32_t(((uint64_t(d.M) + BM - 1) / BM) * h.tiles_n);
                kernel<<<blocks, 256, 0, st>>>(h);
            };
            const bool mask = d.p.R * d.p.S <= 32;
#define CONVLOWER_NCHW_CASE(I, BM, BN, BK, ST)                                                     \
    case I:                                                                                        \
        if (mask) launch(conv_nchw_f32_dma_kernel<BM, BN, BK, 2, 2, ST, true>, BM, BN);           \
        else launch(conv_nchw_f32_dma_kernel<BM, BN, BK, 2, 2, ST, false>, BM, BN);               \
        break;
            switch (d.nchw_variant) {
                case 0:
                    if (mask) launch(conv_nchw_f32_dma_kernel<128, 32, 32, 4, 1, 3, true>, 128, 32);
                    else launch(conv_nchw_f32_dma_kernel<128, 32, 32, 4, 1, 3, false>, 128, 32);
                    break;
                CONVLOWER_NCHW_CASE(1, 128, 64, 32, 3)
                CONVLOWER_NCHW_CASE(2, 128, 128, 32, 3)
                CONVLOWER_NCHW_CASE(3, 64, 128, 32, 3)
                CONVLOWER_NCHW_CASE(4, 128, 64, 16, 4)
                CONVLOWER_NCHW_CASE(5, 128, 64, 16, 6)
                CONVLOWER_NCHW_CASE(6, 64, 64, 32, 4)
                CONVLOWER_NCHW_CASE(7, 64, 64, 16, 6)
                case 8:
                    if (mask) launch(conv_nchw_f32_dma_kernel<128, 32, 16, 4, 1, 4, true>, 128, 32);
                    else launch(conv_nchw_f32_dma_kernel<128, 32, 16, 4, 1, 4, false>, 128, 32);
                    break;
                default: break;
            }
#undef CONVLOWER_NCHW_CASE
        }
        return;
    }
    if (d.dma) {
        switch (d.tile) {
            case TILE_256x128: launch_dma_tile<T, 256, 128, BK, 2, 2, 3>(d, g, st); break;
            case TILE_128x128: launch_dma_tile<T, 128, 128, BK, 2, 2, 4>(d, g, st); break;
            case TILE_128x64: launch_dma_tile<T, 128, 64, BK, 2, 2, 4>(d, g, st); break;
            default: launch_dma_tile<T, 128, 32, BK, 4, 1, 4>(d, g, st); break;
        }
        return;
    }
    switch (d.tile) {
        case TILE_128x128: launch_gemm_tile<T, 128, 128, BK, 2, 2>(d, g, st); break;
        case TILE_128x64: launch_gemm_tile<T, 128, 64, BK, 2, 2>(d, g, st); break;
        default: launch_gemm_tile<T, 128, 32, BK, 4, 1>(d, g, st); break;
    }
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
                    hipStream_t st) {
        launch_gemm<T>(d, x, w, bias, y, ws, st);
    }
};

conv_status_t launch_status() { return from_hip(hipGetLastError()); }

conv_status_t check_ws(const conv_desc& d, const void* ws) {
    if (d.ws_bytes == 0) return CONV_OK;
    return check_dev(ws, 16);
}

// Unchecked stage launches (pointers already validated by the caller).
conv_status_t run_pack(const conv_desc& d, const void* w, void* ws, hipStream_t st) {
    if (!d.pack || d.p.N == 0) return CONV_OK;
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
    by_dtype<GemmOp>(d.p.dtype, d, x, w, bias, y, ws, st);
    return launch_status();
}

}  // namespace

// ====================================================================== C ABI

extern "C" {

conv_status_t conv_create_desc(const conv_params_t* p, conv_desc_t* out) {
    if (!p || !out) return CONV_ERR_NULL_PTR;
    *out = nullptr;
    conv_desc tmp{};
    tmp.p = *p;
    conv_status_t s = plan(*p, tmp);
    if (s != CONV_OK) return s;
    conv_desc* d = new (std::nothrow) conv_desc(tmp);
    if (!d) return CONV_ERR_OOM;
    d->magic = kDescMagic;
    *out = d;
    return CONV_OK;
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
    *info = i;
    return CONV_OK;
}

conv_status_t conv_pack_filter(conv_desc_t d, const void* w, void* ws, void* stream) {
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
    if (!d->pack || d->p.N == 0) return CONV_OK;
    conv_status_t s;
    if ((s = check_dev(w, 16)) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    return run_pack(*d, w, ws, static_cast<hipStream_t>(stream));
}

conv_status_t conv_lower_input(conv_desc_t d, const void* x, void* ws, void* stream) {
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
    if (d->elided || d->p.N == 0) return CONV_OK;
    conv_status_t s;
    if ((s = check_dev(x, 16)) != CONV_OK) return s;
    if ((s = check_ws(*d, ws)) != CONV_OK) return s;
    return run_lower(*d, x, ws, static_cast<hipStream_t>(stream));
}

conv_status_t conv_contract(conv_desc_t d, const void* x, const void* w, const void* bias, void* y, const void* ws,
                            void* stream) {
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
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
    if (!desc_ok(d)) return CONV_ERR_INVALID_ARG;
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
