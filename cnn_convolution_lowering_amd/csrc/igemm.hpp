// The contraction Y[M x K] = A[M x Kc] * B[K x Kc]^T on gfx950 MFMA, with
// the bias add, rounding and NCHW / NHWC store fused into its epilogue.
//
// "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
// Extension", section "Transforming Conv2D into im2col and GEMM": output
// matrix = filter matrix x lowered input; section "Global Memory and Shared
// Memory": reusable tiles are staged in on-chip memory and reused by the
// threads of a block.  A 256-thread workgroup owns a BM x BN output tile; its
// A (input windows) and B (filter) tiles are staged through LDS in two
// buffers, so the global loads of tile k+1 are in flight while the MFMAs
// consume tile k.  LDS tiles are unpadded rows of BK elements whose 16-byte
// chunks are XOR-swizzled by row (see swz_chunk), so that both the tile
// writes and the MFMA fragment reads are free of bank conflicts.
//
// Where the A tile comes from is a loader policy:
//  - StridedRows: rows of a lowered buffer -- im2win strips (a row (n,p,q)
//    starts at n*sN + p*sP + q*sQ; element kk sits (kk / RCp)*sS + kk % RCp
//    past it), explicit im2col rows, or a 1x1 NHWC input read in place;
//  - WindowVecNHWC / WindowElem: the window of output pixel (n,p,q) gathered
//    straight from x, zero outside the image, in the filter's natural
//    contraction order ((r,s,c) for NHWC / KRSC, (c,r,s) for NCHW / KCRS), so
//    no lowered buffer is written at all: the window tile exists only in LDS
//    ("Enabling Memory-efficient Im2win Convolution with Multi-precision
//    Support on GPU CUDA and Tensor Cores", abstract: asynchronous data
//    movement, reduced memory).
//
// MFMA: v_mfma_f32_16x16x32_{f16,bf16} for 16-bit storage, four
// v_mfma_f32_16x16x4_f32 per 16-deep step for fp32 (full fp32 products, no
// reduced-precision inputs); accumulation always in fp32.  Every lane feeds A
// and B with the same k assignment (lane group g holds k = g*VEC .. g*VEC+VEC-1
// of the step), so the sum over k is exact whatever order the hardware uses
// inside one instruction.
#pragma once

#include "device_common.hpp"

namespace convlower {

struct GemmArgs {
    const void* a;      // lowered buffer, or x for the window loaders
    const void* b;      // filter rows [K][ldb]
    const void* bias;   // NULL: no bias
    void* y;
    int64_t M;          // output pixels N*P*Q
    int32_t K;          // output channels
    int32_t Kc;         // contraction length (lowered Kl, or C*R*S for the window loaders)
    int32_t PQ, Q;      // decode m -> (n, p, q)
    int64_t sN, sP, sQ; // StridedRows: row offset (elements)
    int32_t RCp, sS;    // StridedRows: column offset
    int32_t ldb;        // filter row pitch (elements)
    int32_t tiles_n;    // ceil(K / BN)
    int32_t tile_rows;  // output rows per workgroup (fp32 NCHW small-window kernel)
    // ConvLSTM step epilogue: y is h_t; c_prev / c_out the cell states
    // (NCHW, lstm_kh channels); 0 for an ordinary convolution.
    const void* c_prev;
    void* c_out;
    int32_t lstm_kh;
    // Split contraction: ksplit > 1 workgroups per output tile (blockIdx.y),
    // each storing fp32 partial sums in the output layout at part + z*M*K.
    int32_t ksplit;
    void* part;
    // Order in which the pipelined kernel's workgroups take the (split,
    // output tile) pairs: TileOrder.
    int32_t tile_order;
    // window loaders: the convolution itself
    int32_t C, H, W, R, S;
    int32_t sh, sw, ph, pw, dh, dw;
};

// Workgroup -> (split z, tile row, tile column) of the pipelined kernel.
// The GPU deals workgroups to its eight XCDs (each with its own L2) round
// robin by linear index, so in the plain order consecutive tiles, which share
// an input panel, land on different XCDs.  The other orders give each XCD one
// contiguous range of the (z, tile row, tile column) sequence, so that the
// tiles an XCD runs at once share input and filter panels in its L2:
//   TILE_ORDER_XCD_ROWS     the range in row-major order (tile column fastest);
//   TILE_ORDER_XCD_SERPENT  the same, odd tile rows taken right to left, so
//                           that consecutive tiles always share a panel;
//   TILE_ORDER_XCD_COLS     the range in column-major order (tile row fastest).
// ("Enabling Memory-efficient Im2win Convolution ...", abstract: the order
// of memory accesses as a tuning dimension; "GPU-Accelerating MSCRED ...",
// section "Future Work": further tile and thread-block configurations.)
enum TileOrder : int32_t { TILE_ORDER_LINEAR = 0, TILE_ORDER_XCD_ROWS = 1, TILE_ORDER_XCD_SERPENT = 2,
                           TILE_ORDER_XCD_COLS = 3 };
constexpr int kTileOrders = 4;
constexpr int kXcds = 8;

struct TileCoord {
    int m, n, z;
};

__device__ __forceinline__ TileCoord tile_coord(const GemmArgs& g, int tiles_m) {
    const int tiles = tiles_m * g.tiles_n;
    int pos = int(blockIdx.x) + int(blockIdx.y) * int(gridDim.x);
    if (g.tile_order != TILE_ORDER_LINEAR) {
        const int total = tiles * int(gridDim.y);
        const int x = pos % kXcds, i = pos / kXcds;
        const int q = total / kXcds, r = total - q * kXcds;
        pos = x * q + (x < r ? x : r) + i;   // XCD x: [x*q + min(x, r), +q + (x < r))
    }
    TileCoord c;
    c.z = pos / tiles;
    const int t = pos - c.z * tiles;
    if (g.tile_order == TILE_ORDER_XCD_COLS) {
        c.n = t / tiles_m;
        c.m = t - c.n * tiles_m;
    } else {
        c.m = t / g.tiles_n;
        c.n = t - c.m * g.tiles_n;
        if (g.tile_order == TILE_ORDER_XCD_SERPENT && (c.m & 1)) c.n = g.tiles_n - 1 - c.n;
    }
    return c;
}

template <typename T>
struct Mfma;

template <>
struct Mfma<_Float16> {
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

template <>
struct Mfma<__bf16> {
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};

template <>
struct Mfma<float> {
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        // Reinterpret the whole vector, then index it: a bit-cast of one
        // vector element (a[j]) was compiled to element 0 for every j.
        const f32x4 af = __builtin_bit_cast(f32x4, a);
        const f32x4 bf = __builtin_bit_cast(f32x4, b);
#pragma unroll
        for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(af[j], bf[j], c, 0, 0, 0);
        return c;
    }
};

// Output pixel m -> (n, p, q); M < 2^31 is checked on the host.
__device__ __forceinline__ void decode_m(const GemmArgs& g, int32_t m, int32_t& n, int32_t& p, int32_t& q) {
    n = m / g.PQ;
    const int32_t pq = m - n * g.PQ;
    p = pq / g.Q;
    q = pq - p * g.Q;
}

// Position of 16-byte chunk `chunk` of LDS tile row `row` (CPR chunks per row).
// Measured on gfx950: a ds_read_b128 is served 16 lanes per cycle over 64
// four-byte banks, the lanes grouped by bits 3 and 5 of the lane id (lanes
// 0-7 with 16-23, ...); a ds_write_b128 is served 8 consecutive lanes per
// cycle over 32 banks.  A fragment read (lane l: row l%16, chunk l/16 of the
// step) then puts rows r and r+4 (64-byte rows) or r and r+2 (128-byte rows)
// on the same banks unless their chunks are moved apart; XOR-ing the chunk
// index with ((row >> 1) & 3), scaled to keep chunk pairs together in
// 128-byte rows, separates them, and keeps the row-major tile writes (8
// lanes covering 128 contiguous bytes) conflict-free as well.
//
// SWZ = 1 is the variant for 32 x 32 fragments (lane l: row l%32, chunk
// l/32): one read cycle then covers rows 0-7 and 16-23 (or 8-15 and 24-31) of
// a single chunk, so rows 16 apart must land on different banks as well as
// rows 4 (64-byte rows) or 2 (128-byte rows) apart; the XOR takes bits 2 and
// 4 of the row (64-byte rows) or bits 1, 2 and 4 (128-byte rows).  It depends
// on row bits 0-4 only, like SWZ = 0.
template <int CPR, int SWZ = 0>
__device__ __forceinline__ int swz_chunk(int row, int chunk) {
    static_assert(CPR == 4 || CPR == 8, "tile rows of 64 or 128 bytes");
    if constexpr (SWZ == 0)
        return CPR == 4 ? (chunk ^ ((row >> 1) & 3)) : (chunk ^ (((row >> 1) & 3) << 1));
    else
        return CPR == 4 ? (chunk ^ (((row >> 2) & 1) | (((row >> 4) & 1) << 1)))
                        : (chunk ^ (((row >> 1) & 3) | (((row >> 4) & 1) << 2)));
}

// ---------------------------------------------------------------------------
// Loaders.  Each holds NV 16-byte registers of the next tile: fetch() issues
// the global loads for the current contraction position, next() moves it by
// BK, put() writes the registers into an LDS tile of ROWS rows of BK elements
// (chunks placed by swz_chunk).

// Rows of a strided matrix, 16-byte vectors along the contraction (k-fast
// mapping: consecutive threads take consecutive vectors of a row).  Rows are
// output pixels for the A side (PIXELS) or filter rows for the B side.  With
// SEGMENTED the column offset is (kk / RCp)*sS + kk % RCp (im2win strips);
// otherwise it is kk.  ELEM gathers a vector element by element, for row
// pitches that are not whole vectors.
template <typename T, int ROWS, int BK, bool SEGMENTED, bool ELEM>
struct StridedRows {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int KV = BK / VEC;
    static constexpr int NV = (ROWS * KV + 255) / 256;
    static_assert(256 % KV == 0, "tile depth");
    u32x4 r[NV];
    int64_t off[NV];
    bool ok[NV];
    int kv, kk, t;
    int64_t seg;

    template <bool PIXELS>
    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        kv = tid % KV;
        kk = kv * VEC;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * 256;
            const int64_t row = row0 + v / KV;
            if (PIXELS) {
                ok[i] = (v < ROWS * KV) && (row < g.M);
                int32_t n, p, q;
                decode_m(g, ok[i] ? int32_t(row) : 0, n, p, q);
                off[i] = int64_t(n) * g.sN + int64_t(p) * g.sP + int64_t(q) * g.sQ;
            } else {
                ok[i] = (v < ROWS * KV) && (row < g.K);
                off[i] = (ok[i] ? row : 0) * int64_t(g.ldb);
            }
        }
        if (SEGMENTED) {
            t = kk % g.RCp;
            seg = int64_t(kk / g.RCp) * g.sS;
        } else {
            t = kk;
            seg = 0;
        }
    }
    __device__ __forceinline__ void fetch(const GemmArgs& g, const T* __restrict__ base) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            if (!ELEM) {
                r[i] = (ok[i] && kk < g.Kc) ? load16(base + off[i] + seg + t) : zero4();
            } else {
                // element by element; a vector may cross into the next
                // segment (the next tap's columns of an unpadded strip)
                Pack16<T> pk;
                int tt = t;
                int64_t sg = seg;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    if (SEGMENTED)
                        while (tt >= g.RCp) {
                            tt -= g.RCp;
                            sg += g.sS;
                        }
                    pk.e[e] = (ok[i] && kk + e < g.Kc) ? base[off[i] + sg + tt] : T(0);
                    ++tt;
                }
                r[i] = pk.v;
            }
        }
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        t += BK;
        if (SEGMENTED) {
            while (t >= g.RCp) {
                t -= g.RCp;
                seg += g.sS;
            }
        }
    }
    __device__ __forceinline__ void put(T* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * 256;
            const int row = v / KV;
            if (v < ROWS * KV) store16(lds + row * BK + swz_chunk<KV>(row, kv) * VEC, r[i]);
        }
    }
};

// Window of each output pixel gathered from NHWC x, 16-byte vectors of
// channels (C a whole number of vectors), contraction order (r, s, c).
template <typename T, int ROWS, int BK>
struct WindowVecNHWC {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int KV = BK / VEC;
    static constexpr int NV = (ROWS * KV + 255) / 256;
    static_assert(256 % KV == 0, "tile depth");
    u32x4 r[NV];
    int64_t nbase[NV];
    int32_t h0[NV], w0[NV];
    bool ok[NV];
    int kv, kk, c0, s, rr;

    template <bool PIXELS>
    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        static_assert(PIXELS, "window loaders feed the pixel side");
        kv = tid % KV;
        kk = kv * VEC;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * 256;
            const int64_t m = row0 + v / KV;
            ok[i] = (v < ROWS * KV) && (m < g.M);
            int32_t n, p, q;
            decode_m(g, ok[i] ? int32_t(m) : 0, n, p, q);
            nbase[i] = int64_t(n) * g.H * g.W * g.C;
            h0[i] = p * g.sh - g.ph;
            w0[i] = q * g.sw - g.pw;
        }
        c0 = kk % g.C;
        const int rs = kk / g.C;
        s = rs % g.S;
        rr = rs / g.S;
    }
    __device__ __forceinline__ void fetch(const GemmArgs& g, const T* __restrict__ x) {
        const int dh = rr * g.dh, dw = s * g.dw;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int h = h0[i] + dh, w = w0[i] + dw;
            const bool in = ok[i] && kk < g.Kc && unsigned(h) < unsigned(g.H) && unsigned(w) < unsigned(g.W);
            r[i] = in ? load16(x + nbase[i] + (int64_t(h) * g.W + w) * g.C + c0) : zero4();
        }
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        c0 += BK;
        while (c0 >= g.C) {
            c0 -= g.C;
            if (++s == g.S) {
                s = 0;
                ++rr;
            }
        }
    }
    __device__ __forceinline__ void put(T* lds, int tid) const {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int v = tid + i * 256;
            const int row = v / KV;
            if (v < ROWS * KV) store16(lds + row * BK + swz_chunk<KV>(row, kv) * VEC, r[i]);
        }
    }
};

// Window of each output pixel gathered element by element (NCHW input, or
// NHWC with C not a whole number of vectors).  Pixel-fast mapping: the
// threads of a wave take consecutive output pixels, so for one contraction
// element their loads walk along an input row; each thread takes EPT
// consecutive contraction elements of its pixel.  Order (c, r, s) for NCHW,
// (r, s, c) for NHWC -- the filter's own order.
template <typename T, int ROWS, int BK, bool NHWC>
struct WindowElem {
    static constexpr int VEC = Vec<T>::n;
    static constexpr int TPR = 256 / ROWS;        // threads per pixel row
    static constexpr int EPT = BK / TPR;          // elements per thread
    static constexpr int NV = EPT / VEC;
    static_assert(256 % ROWS == 0 && BK % TPR == 0 && EPT % VEC == 0, "window tile shape");
    u32x4 r[NV];
    int64_t nbase;
    int32_t h0, w0;
    bool ok;
    int row, kq, kk;       // kk: first contraction element of this thread
    int c, rr, s;          // its decoded position

    __device__ __forceinline__ void decode(const GemmArgs& g) {
        if (NHWC) {
            c = kk % g.C;
            const int rs = kk / g.C;
            s = rs % g.S;
            rr = rs / g.S;
        } else {
            const int RS = g.R * g.S;
            c = kk / RS;
            const int rs = kk - c * RS;
            rr = rs / g.S;
            s = rs - rr * g.S;
        }
    }
    template <bool PIXELS>
    __device__ __forceinline__ void init(const GemmArgs& g, int64_t row0, int tid) {
        static_assert(PIXELS, "window loaders feed the pixel side");
        row = tid % ROWS;
        kq = tid / ROWS;
        const int64_t m = row0 + row;
        ok = m < g.M;
        int32_t n, p, q;
        decode_m(g, ok ? int32_t(m) : 0, n, p, q);
        nbase = int64_t(n) * g.C * g.H * g.W;
        h0 = p * g.sh - g.ph;
        w0 = q * g.sw - g.pw;
        kk = kq * EPT;
        decode(g);
    }
    __device__ __forceinline__ void fetch(const GemmArgs& g, const T* __restrict__ x) {
        int cc = c, r2 = rr, s2 = s;
        Pack16<T> pk[NV];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int h = h0 + r2 * g.dh, w = w0 + s2 * g.dw;
            T val = T(0);
            if (ok && kk + e < g.Kc && unsigned(h) < unsigned(g.H) && unsigned(w) < unsigned(g.W)) {
                const int64_t o = NHWC ? (int64_t(h) * g.W + w) * g.C + cc : (int64_t(cc) * g.H + h) * g.W + w;
                val = x[nbase + o];
            }
            pk[e / VEC].e[e % VEC] = val;
            if (NHWC) {
                if (++cc == g.C) {
                    cc = 0;
                    if (++s2 == g.S) {
                        s2 = 0;
                        ++r2;
                    }
                }
            } else {
                if (++s2 == g.S) {
                    s2 = 0;
                    if (++r2 == g.R) {
                        r2 = 0;
                        ++cc;
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NV; ++j) r[j] = pk[j].v;
    }
    __device__ __forceinline__ void next(const GemmArgs& g) {
        kk += BK;
        decode(g);
    }
    __device__ __forceinline__ void put(T* lds, int) const {
#pragma unroll
        for (int j = 0; j < NV; ++j) store16(lds + row * BK + swz_chunk<BK / VEC>(row, kq * NV + j) * VEC, r[j]);
    }
};

// ConvLSTM step epilogue (fp32, NCHW), one cell update per output element;
// "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
// Extension" names the ConvLSTM stage without equations, read here as the
// standard peephole-free cell: with the gates z = acc + bias,
//     c_t = sigmoid(z_f) * c_prev + sigmoid(z_i) * tanh(z_g)
//     h_t = sigmoid(z_o) * tanh(c_t).
// The tile is BN = 64 packed gate rows (see PackArgs::lstm_kh) seen by one
// wave (WN = 64): block j of the lane's accumulators is gate j (i, f, g, o)
// of hidden channel n0/4 + (lane & 15), pixels m .. m+3.
__device__ __forceinline__ float sigmoid_f32(float z) { return 1.0f / (1.0f + expf(-z)); }

template <int WM, int TM, int TN>
__device__ __forceinline__ void lstm_store_tile(const GemmArgs& g, const f32x4 (&acc)[TM][TN], int64_t m0, int n0,
                                                int wm, int lane) {
    static_assert(TN == 4, "one 16-column block per gate");
    const int kh = g.lstm_kh;
    const int hid = n0 / 4 + (lane & 15);
    const float* __restrict__ bias = static_cast<const float*>(g.bias);
    float bg[4];
#pragma unroll
    for (int gt = 0; gt < 4; ++gt) bg[gt] = bias ? bias[gt * kh + hid] : 0.f;
    const float* __restrict__ cp = static_cast<const float*>(g.c_prev);
    float* __restrict__ co = static_cast<float*>(g.c_out);
    float* __restrict__ ho = static_cast<float*>(g.y);
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t mb = m0 + wm * WM + i * 16 + 4 * (lane >> 4);
        if (mb >= g.M) continue;
        float cv[4], hv[4], cprev[4];
        const bool vec = (g.PQ & 3) == 0;   // then mb % 4 == 0: four pixels of one image, contiguous
        int64_t off[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int64_t m = mb + e < g.M ? mb + e : mb;
            const int32_t n = int32_t(m / g.PQ);
            off[e] = (int64_t(n) * kh + hid) * g.PQ + (m - int64_t(n) * g.PQ);
        }
        if (vec) {
            const f32x4 c4 = __builtin_bit_cast(f32x4, load16(cp + off[0]));
#pragma unroll
            for (int e = 0; e < 4; ++e) cprev[e] = c4[e];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) cprev[e] = cp[off[e]];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float zi = acc[i][0][e] + bg[0], zf = acc[i][1][e] + bg[1];
            const float zg = acc[i][2][e] + bg[2], zo = acc[i][3][e] + bg[3];
            cv[e] = sigmoid_f32(zf) * cprev[e] + sigmoid_f32(zi) * tanhf(zg);
            hv[e] = sigmoid_f32(zo) * tanhf(cv[e]);
        }
        if (vec) {
            store16(co + off[0], u32x4{__float_as_uint(cv[0]), __float_as_uint(cv[1]), __float_as_uint(cv[2]),
                                       __float_as_uint(cv[3])});
            store16(ho + off[0], u32x4{__float_as_uint(hv[0]), __float_as_uint(hv[1]), __float_as_uint(hv[2]),
                                       __float_as_uint(hv[3])});
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (mb + e >= g.M) break;
                co[off[e]] = cv[e];
                ho[off[e]] = hv[e];
            }
        }
    }
}

// Epilogue shared by the contraction kernels: y = round(acc + bias[k]),
// stored in NPQK (NHWC_OUT) or NKPQ order.
template <typename T, int BM, int BN, int WM, int WN, int TM, int TN, bool NHWC_OUT>
__device__ __forceinline__ void store_tile(const GemmArgs& g, const f32x4 (&acc)[TM][TN], int64_t m0, int n0, int wm,
                                           int wn, int lane) {
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    if (NHWC_OUT) {
        // acc[i][j][e]: channel n0 + wn*WN + j*16 + 4*(lane>>4) + e, pixel m0 + wm*WM + i*16 + (lane&15)
        float bv[TN][4];   // this lane's bias values, loaded once
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int k = n0 + wn * WN + j * 16 + 4 * (lane >> 4) + e;
                bv[j][e] = (bias && k < g.K) ? to_f32(bias[k]) : 0.f;
            }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = m0 + wm * WM + i * 16 + (lane & 15);
            if (m >= g.M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int k = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e] + bv[j][e];
                T* dst = y + m * g.K + k;
                if (k + 3 < g.K && (g.K & 3) == 0) {
                    if (sizeof(T) == 4) {
                        store16(dst, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                           __float_as_uint(v[3])});
                    } else {
                        union {
                            u32x2 u;
                            T e[4];
                        } pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(v[e]);
                        *reinterpret_cast<u32x2*>(dst) = pk.u;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (k + e < g.K) dst[e] = from_f32<T>(v[e]);
                }
            }
        }
    } else {
        // acc[i][j][e]: pixel m0 + wm*WM + i*16 + 4*(lane>>4) + e, channel n0 + wn*WN + j*16 + (lane&15)
        float bv[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int k = n0 + wn * WN + j * 16 + (lane & 15);
            bv[j] = (bias && k < g.K) ? to_f32(bias[k]) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int k = n0 + wn * WN + j * 16 + (lane & 15);
            if (k >= g.K) continue;
            const float bk = bv[j];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int64_t mb = m0 + wm * WM + i * 16 + 4 * (lane >> 4);
                if (mb >= g.M) continue;
                if ((g.PQ & 3) == 0) {
                    // mb % 4 == 0 and PQ % 4 == 0: the 4 pixels are in one image and
                    // contiguous in NKPQ, so one 16-byte (fp32) or 8-byte store
                    const int32_t n = int32_t(mb) / g.PQ;
                    const int32_t pq = int32_t(mb) - n * g.PQ;
                    T* dst = y + (int64_t(n) * g.K + k) * g.PQ + pq;
                    if (sizeof(T) == 4) {
                        store16(dst, u32x4{__float_as_uint(acc[i][j][0] + bk), __float_as_uint(acc[i][j][1] + bk),
                                           __float_as_uint(acc[i][j][2] + bk), __float_as_uint(acc[i][j][3] + bk)});
                    } else {
                        union {
                            u32x2 u;
                            T e[4];
                        } pk;
#pragma unroll
                        for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(acc[i][j][e] + bk);
                        *reinterpret_cast<u32x2*>(dst) = pk.u;
                    }
                    continue;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int64_t m = mb + e;
                    if (m >= g.M) break;
                    const int32_t n = int32_t(m) / g.PQ;
                    const int32_t pq = int32_t(m) - n * g.PQ;
                    y[(int64_t(n) * g.K + k) * g.PQ + pq] = from_f32<T>(acc[i][j][e] + bk);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// BM x BN output tile, BK-deep LDS stages, WGM x WGN waves (4 in all).
// NHWC_OUT: the MFMA is fed (filter, pixel) so a lane ends with 4 consecutive
// output channels of one pixel (contiguous in NPQK); otherwise (pixel, filter)
// so a lane ends with 4 consecutive pixels of one channel (contiguous in NKPQ).
template <typename T, int BM, int BN, int BK, int WGM, int WGN, bool NHWC_OUT, class ALoad, class BLoad>
__global__ void __launch_bounds__(256) conv_gemm_kernel(GemmArgs g) {
    constexpr int VEC = Vec<T>::n;
    constexpr int CPR = BK / VEC;     // 16-byte chunks per LDS tile row
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int KB = 4 * VEC;       // contraction depth of one fragment step
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    static_assert(BK % KB == 0, "tile depth");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");

    __shared__ __attribute__((aligned(16))) T sA[2][BM * BK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile_m = blockIdx.x / g.tiles_n;
    const int tile_n = blockIdx.x - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    const T* __restrict__ A = static_cast<const T*>(g.a);
    const T* __restrict__ B = static_cast<const T*>(g.b);

    ALoad la;
    BLoad lb;
    la.template init<true>(g, m0, tid);
    lb.template init<false>(g, n0, tid);

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = (g.Kc + BK - 1) / BK;
    la.fetch(g, A);
    lb.fetch(g, B);
    la.put(sA[0], tid);
    lb.put(sB[0], tid);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_chunk = lane >> 4;
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {
            la.next(g);
            lb.next(g);
            la.fetch(g, A);
            lb.fetch(g, B);
        }
#pragma unroll
        for (int kb = 0; kb < BK / KB; ++kb) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm * WM + i * 16 + frag_row;
                fa[i] = load16(&sA[cur][row * BK + swz_chunk<CPR>(row, kb * 4 + frag_chunk) * VEC]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn * WN + j * 16 + frag_row;
                fb[j] = load16(&sB[cur][row * BK + swz_chunk<CPR>(row, kb * 4 + frag_chunk) * VEC]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = NHWC_OUT ? Mfma<T>::run(fb[j], fa[i], acc[i][j]) : Mfma<T>::run(fa[i], fb[j], acc[i][j]);
        }
        if (more) {
            la.put(sA[cur ^ 1], tid);
            lb.put(sB[cur ^ 1], tid);
        }
        __syncthreads();
    }

    store_tile<T, BM, BN, WM, WN, TM, TN, NHWC_OUT>(g, acc, m0, n0, wm, wn, lane);
}

}  // namespace convlower
