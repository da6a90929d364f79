// Lowering kernels: window strips (im2win), explicit im2col rows, filter pack.
//
// Both lowered layouts order one contraction row as (s, r, c): for kernel
// column s, the R*C values x[h_r][w_s][c] of one padded input column, padded
// with zeros to RCp = R*C rounded up to a whole 16-byte vector.
//
//  im2win  Win[n][p][j][t], t < RCp: input column w = j - pw of the R input
//          rows h = p*sh - ph + r*dh, for the W_used columns j the windows of
//          output row p touch.  A contraction row (n, p, q) is the S strip
//          columns j = q*sw + s*dw, so overlapping windows share storage and
//          (for dw = 1) a row is one contiguous run -- the window layout of
//          "Enabling Memory-efficient Im2win Convolution with Multi-precision
//          Support on GPU CUDA and Tensor Cores" (abstract).
//  im2col  Col[m = (n,p,q)][s*RCp + t]: one materialised row per output pixel,
//          the explicit matrix of overlapping windows of "GPU-Accelerating
//          MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch Extension",
//          section "Transforming Conv2D into im2col and GEMM".
//
// Zero padding of the convolution is written into the lowered buffer, so the
// contraction never tests bounds on the input.
#pragma once

#include "device_common.hpp"

namespace convlower {

struct LowerArgs {
    const void* x;
    void* out;
    int32_t N, C, H, W;
    int32_t P, Q, R, S;
    int32_t sh, sw, ph, pw, dh, dw;
    int32_t W_used;   // strip columns per (n, p)
    int32_t RCp;      // R*C padded to whole vectors
    int32_t Kl;       // S*RCp
    // NCHW input split over two tensors (a ConvLSTM step's x and h): channels
    // c < C1 come from x (C1 per image), the rest from x2 (C - C1 per image).
    // C1 == C and x2 == nullptr for an ordinary convolution.
    const void* x2;
    int32_t C1;
    // Band kernels: an item is (image, band of G output rows, chunk of CW
    // output columns -- strip columns for im2win, q for im2col); it stages
    // BR input rows of TW tile columns at LDS row pitch WL elements (and,
    // NCHW, channel pitch CS elements).
    int32_t G, CW, BR, TW, WL, CS;
    FastDiv fd_cb;    // column chunks per band
    FastDiv fd_pb;    // bands per image
    FastDiv fd_tw;    // staging: elements (NCHW) or vectors (NHWC) per staged row
    FastDiv fd_br;    // staging: rows per channel (NCHW)
    FastDiv fd_row;   // output vectors per output row of the band: CW * fd_vpc.d
    FastDiv fd_vpc;   // output vectors per output column: RCp/VEC (im2win) or Kl/VEC (im2col)
    FastDiv fd_cpv;   // RCp/VEC
    FastDiv fd_c;     // C
    FastDiv fd_p;     // P
    FastDiv fd_q;     // Q
    FastDiv fd_nv;    // NCHW vector staging: 16-byte vectors per channel's band of rows (bound)
    FastDiv fd_w;     // W
};

// x element (n, c, h, w) in either layout, zero outside the image.
template <typename T, bool NHWC>
__device__ __forceinline__ T x_at(const LowerArgs& a, const T* __restrict__ x, int n, int c, int h, int w) {
    if (h < 0 || h >= a.H || w < 0 || w >= a.W) return T(0);
    if (!NHWC && c >= a.C1)
        return static_cast<const T*>(a.x2)[((int64_t(n) * (a.C - a.C1) + (c - a.C1)) * a.H + h) * a.W + w];
    int64_t off = NHWC ? ((int64_t(n) * a.H + h) * a.W + w) * a.C + c
                       : ((int64_t(n) * a.C1 + c) * a.H + h) * a.W + w;
    return x[off];
}

// ---------------------------------------------------------------------------
// im2win and im2col, NHWC input with C a whole number of 16-byte vectors: a
// vector of the lowered row is a vector of one x row, so the copy is 16-byte
// load -> 16-byte store.  Each thread moves LOWER_U vectors LOWER_U*256 apart,
// all loads issued before the first store; outside the image the load reads
// a clamped in-image address and the value is replaced by zeros, so no load
// is conditional.
constexpr int LOWER_U = 4;

// Lowered vector v of strip (n, p): strip column j, elements t0.. of R*C.
template <typename T>
__device__ __forceinline__ const T* nhwc_src(const LowerArgs& a, const T* x, int n, int p, int wcol, int t0,
                                             bool& in) {
    const int r = int(fdiv(uint32_t(t0), a.fd_c));
    const int c0 = t0 - r * a.C;
    const int h = p * a.sh - a.ph + r * a.dh;
    in = h >= 0 && h < a.H && wcol >= 0 && wcol < a.W;
    const int hc = min(max(h, 0), a.H - 1), wc = min(max(wcol, 0), a.W - 1);
    return x + ((int64_t(n) * a.H + hc) * a.W + wc) * a.C + c0;
}

// grid.x = N*P strips, grid.y = ceil(W_used*RCp/VEC / (256*LOWER_U)).
template <typename T>
__global__ void __launch_bounds__(256) im2win_nhwc_vec_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    const int strip = blockIdx.x;
    const int n = int(fdiv(uint32_t(strip), a.fd_p)), p = strip - n * a.P;
    const uint32_t vps = uint32_t(a.W_used) * a.fd_cpv.d;   // vectors per strip
    const T* __restrict__ x = static_cast<const T*>(a.x);
    T* out = static_cast<T*>(a.out) + int64_t(strip) * a.W_used * a.RCp;
    u32x4 val[LOWER_U];
    bool live[LOWER_U];
#pragma unroll
    for (int u = 0; u < LOWER_U; ++u) {
        const uint32_t v = (blockIdx.y * LOWER_U + u) * 256 + threadIdx.x;
        live[u] = v < vps;
        const uint32_t vv = live[u] ? v : 0;
        const int j = int(fdiv(vv, a.fd_cpv));
        const int t0 = int(vv - uint32_t(j) * a.fd_cpv.d) * VEC;
        bool in;
        const T* src = nhwc_src<T>(a, x, n, p, j - a.pw, t0, in);
        val[u] = load16(src);
        if (!in) val[u] = zero4();
    }
#pragma unroll
    for (int u = 0; u < LOWER_U; ++u) {
        const uint32_t v = (blockIdx.y * LOWER_U + u) * 256 + threadIdx.x;
        if (live[u]) store16(out + int64_t(v) * VEC, val[u]);
    }
}

// Grid-stride over the M*Kl/VEC vectors of Col (checked on the host to stay
// below 2^31), LOWER_U vectors per thread and pass.
template <typename T>
__global__ void __launch_bounds__(256) im2col_nhwc_vec_kernel(LowerArgs a, uint32_t total_vec) {
    constexpr int VEC = Vec<T>::n;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    T* out = static_cast<T*>(a.out);
    const uint32_t step = gridDim.x * 256u * LOWER_U;
    for (uint32_t base = blockIdx.x * 256u * LOWER_U + threadIdx.x; base < total_vec; base += step) {
        u32x4 val[LOWER_U];
#pragma unroll
        for (int u = 0; u < LOWER_U; ++u) {
            const uint32_t v0 = base + u * 256u;
            const uint32_t v = v0 < total_vec ? v0 : 0;
            const uint32_t m = fdiv(v, a.fd_vpc);                  // Col row (n, p, q)
            const uint32_t kv = v - m * a.fd_vpc.d;
            const uint32_t s = fdiv(kv, a.fd_cpv);
            const int t0 = int(kv - s * a.fd_cpv.d) * VEC;
            const uint32_t np = fdiv(m, a.fd_q);
            const int q = int(m - np * a.fd_q.d);
            const int n = int(fdiv(np, a.fd_p)), p = int(np) - n * a.P;
            bool in;
            const T* src = nhwc_src<T>(a, x, n, p, q * a.sw - a.pw + int(s) * a.dw, t0, in);
            val[u] = load16(src);
            if (!in) val[u] = zero4();
        }
#pragma unroll
        for (int u = 0; u < LOWER_U; ++u) {
            const uint32_t v = base + u * 256u;
            if (v < total_vec) store16(out + int64_t(v) * VEC, val[u]);
        }
    }
}

// ---------------------------------------------------------------------------
// Band lowering, for the layouts where a lowered vector is not a vector of
// x: NCHW input (a strip column gathers one element from each of R*C rows)
// and NHWC input whose C is not a whole number of vectors.  An item is an
// image n, a band of G output rows from p0 = pb*G and a chunk of CW output
// columns.  The block first copies the input the item reads into LDS with
// coalesced loads (zeros outside the image), then writes the item's lowered
// rows as whole 16-byte vectors, consecutive lanes on consecutive vectors,
// gathering each vector's elements from LDS.  grid.x = items; dynamic LDS is
// the staged tile.

// Item -> (n, pb, cb).
__device__ __forceinline__ void band_item(const LowerArgs& a, int& n, int& pb, int& cb) {
    const uint32_t item = blockIdx.x;
    const uint32_t ib = fdiv(item, a.fd_cb);
    cb = int(item - ib * a.fd_cb.d);
    n = int(fdiv(ib, a.fd_pb));
    pb = int(ib) - n * int(a.fd_pb.d);
}

// Output vector v of the item -> (pp = output row in the band, col = output
// column in the chunk, s = kernel column (im2col), tv = vector in RCp).
template <bool COL>
__device__ __forceinline__ void band_vector(const LowerArgs& a, uint32_t v, int& pp, int& col, int& s, int& tv) {
    pp = int(fdiv(v, a.fd_row));
    const uint32_t rem = v - uint32_t(pp) * a.fd_row.d;
    col = int(fdiv(rem, a.fd_vpc));
    const uint32_t kv = rem - uint32_t(col) * a.fd_vpc.d;
    if (COL) {
        s = int(fdiv(kv, a.fd_cpv));
        tv = int(kv) - s * int(a.fd_cpv.d);
    } else {
        s = 0;
        tv = int(kv);
    }
}

// NCHW: the tile is tile[c][hh][jj] (row pitch WL, channel pitch CS, both
// odd, so that a wave's reads of every k-th channel spread over banks): input
// row h = p0*sh - ph + hh of channel c, strip column j0 + jj (x column
// j0 + jj - pw), where j0 is the chunk's first strip column.  BR = (G-1)*sh
// + (R-1)*dh + 1 rows; TW = CW strip columns (im2win) or (CW-1)*sw +
// (S-1)*dw + 1 (im2col).
// VLOAD (one chunk spans every column, and every channel plane starts on a
// 16-byte boundary): the band's rows inside the image are one contiguous run
// of each plane, so the tile is zeroed and then filled from 16-byte loads of
// those runs (fd_nv.d vectors cover a run from any start); otherwise element
// loads with the zeros outside the image selected in.
template <typename T, bool COL, bool VLOAD>
__global__ void __launch_bounds__(256) lower_nchw_band_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    constexpr int U = 8;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* tile = reinterpret_cast<T*>(lds_raw);
    int n, pb, cb;
    band_item(a, n, pb, cb);
    const int p0 = pb * a.G;
    const int hlo = p0 * a.sh - a.ph;
    const int j0 = COL ? cb * a.CW * a.sw : cb * a.CW;
    const int64_t plane = int64_t(a.H) * a.W;
    const T* xn = static_cast<const T*>(a.x) + int64_t(n) * a.C1 * plane;
    // channels c >= C1 (a second input only): plane c - C1 of image n there
    const T* x2n = a.x2 ? static_cast<const T*>(a.x2) + int64_t(n) * (a.C - a.C1) * plane : xn;
    const uint32_t stage_total = uint32_t(a.C) * a.BR * a.TW;
    if (VLOAD) {
        const int ha = max(hlo, 0), hb = min(hlo + a.BR, a.H);
        // Zeros where the vector pass below writes nothing (so no barrier
        // between them): every column of the tile rows outside the image --
        // rows outside [lo, hi) -- and, in the rows inside, the columns left
        // of the image ([0, zl)) and right of it ([zr, TW)).
        const int lo = min(ha - hlo, a.BR), hi = max(hb - hlo, lo);
        const int nout = a.BR - (hi - lo);
        for (int i = threadIdx.x; i < a.C * nout * a.TW; i += 256) {
            const int c = i / (nout * a.TW), rem = i - c * nout * a.TW;
            const int r = rem / a.TW, jj = rem - r * a.TW;
            tile[c * a.CS + (r < lo ? r : r - lo + hi) * a.WL + jj] = T(0);
        }
        const int zl = min(a.pw, a.TW), zr = min(a.pw + a.W, a.TW), zc = zl + a.TW - zr;
        for (int i = threadIdx.x; i < a.C * (hi - lo) * zc; i += 256) {
            const int c = i / ((hi - lo) * zc), rem = i - c * (hi - lo) * zc;
            const int r = rem / zc, k = rem - r * zc;
            tile[c * a.CS + (lo + r) * a.WL + (k < zl ? k : zr + k - zl)] = T(0);
        }
        const int fa = ha * a.W, fb = hb * a.W;   // the run of each plane, elements
        const int va = fa / VEC;                  // its first vector
        const uint32_t vtotal = uint32_t(a.C) * a.fd_nv.d;
        for (uint32_t base = threadIdx.x; base < vtotal; base += 256 * 4) {
            u32x4 val[4];
            int f0[4], c4[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t i0 = base + u * 256;
                const uint32_t i = i0 < vtotal ? i0 : 0;
                const int c = int(fdiv(i, a.fd_nv));
                const int v = va + int(i - uint32_t(c) * a.fd_nv.d);
                const bool live = i0 < vtotal && v * VEC < fb;
                const T* plane_c = c < a.C1 ? xn + int64_t(c) * plane : x2n + int64_t(c - a.C1) * plane;
                val[u] = load16(plane_c + (live ? v * VEC : 0));   // not live: the plane's first vector
                f0[u] = live ? v * VEC : -1;
                c4[u] = c;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (f0[u] < 0) continue;
                Pack16<T> pk;
                pk.v = val[u];
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    const int f = f0[u] + e;
                    const int h = int(fdiv(uint32_t(f), a.fd_w));
                    const int jj = f - h * a.W + a.pw;
                    if (f >= fa && f < fb && jj < a.TW) tile[c4[u] * a.CS + (h - hlo) * a.WL + jj] = pk.e[e];
                }
            }
        }
    }
    for (uint32_t base = threadIdx.x; !VLOAD && base < stage_total; base += 256 * U) {
        T val[U];
        int dst[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i0 = base + u * 256;
            const uint32_t i = i0 < stage_total ? i0 : 0;
            const uint32_t row = fdiv(i, a.fd_tw);
            const int jj = int(i - row * a.fd_tw.d);
            const int c = int(fdiv(row, a.fd_br));
            const int hh = int(row) - c * a.BR;
            const int h = hlo + hh, w = j0 + jj - a.pw;
            const bool in = h >= 0 && h < a.H && w >= 0 && w < a.W;
            const int hc = min(max(h, 0), a.H - 1), wc = min(max(w, 0), a.W - 1);
            const T* src =
                (c < a.C1 ? xn + int64_t(c) * plane : x2n + int64_t(c - a.C1) * plane) + int64_t(hc) * a.W + wc;
            val[u] = *src;
            if (!in) val[u] = T(0);
            dst[u] = i0 < stage_total ? c * a.CS + hh * a.WL + jj : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (dst[u] >= 0) tile[dst[u]] = val[u];
    }
    __syncthreads();
    const int RC = a.R * a.C;
    const int cstride = a.CS;
    const uint32_t out_total = uint32_t(a.G) * a.fd_row.d;
    for (uint32_t v = threadIdx.x; v < out_total; v += 256) {
        int pp, col, s, tv;
        band_vector<COL>(a, v, pp, col, s, tv);
        const int p = p0 + pp;
        const int gcol = cb * a.CW + col;
        if (p >= a.P || gcol >= (COL ? a.Q : a.W_used)) continue;
        const int tcol = COL ? col * a.sw + s * a.dw : col;
        const int t0 = tv * VEC;
        int r = int(fdiv(uint32_t(t0), a.fd_c));
        int c = t0 - r * a.C;
        const T* trow = tile + pp * a.sh * a.WL + tcol;
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            pk.e[e] = t0 + e < RC ? trow[c * cstride + r * a.dh * a.WL] : T(0);
            if (++c == a.C) {
                c = 0;
                ++r;
            }
        }
        T* out = static_cast<T*>(a.out) +
                 (COL ? ((int64_t(n) * a.P + p) * a.Q + gcol) * a.Kl + (s * a.RCp + t0)
                      : ((int64_t(n) * a.P + p) * a.W_used + gcol) * a.RCp + t0);
        store16(out, pk.v);
    }
}

// NHWC with C not a whole number of vectors: the tile is BR whole x rows,
// tile[hh][w*C + c] at pitch WL = W*C elements (row h = p0*sh - ph + hh,
// zeros outside the image); a column outside the image gives a zero vector.
// VLOAD: W*C*sizeof(T) and x are 16-byte aligned, so the staging moves
// 16-byte vectors (fd_tw counts vectors per row); otherwise elements.
template <typename T, bool COL, bool VLOAD>
__global__ void __launch_bounds__(256) lower_nhwc_band_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    constexpr int U = VLOAD ? 8 : 16;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* tile = reinterpret_cast<T*>(lds_raw);
    int n, pb, cb;
    band_item(a, n, pb, cb);
    const int p0 = pb * a.G;
    const int hlo = p0 * a.sh - a.ph;
    const T* __restrict__ xn = static_cast<const T*>(a.x) + int64_t(n) * a.H * a.WL;
    const uint32_t stage_total = uint32_t(a.BR) * a.fd_tw.d;
    for (uint32_t base = threadIdx.x; base < stage_total; base += 256 * U) {
        if (VLOAD) {
            u32x4 val[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i0 = base + u * 256;
                const uint32_t i = i0 < stage_total ? i0 : 0;
                const int hh = int(fdiv(i, a.fd_tw));
                const int cv = int(i - uint32_t(hh) * a.fd_tw.d);
                const int h = hlo + hh;
                const int hc = min(max(h, 0), a.H - 1);
                val[u] = load16(xn + int64_t(hc) * a.WL + cv * VEC);
                if (h < 0 || h >= a.H) val[u] = zero4();
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + u * 256;
                if (i < stage_total) store16(tile + int64_t(i) * VEC, val[u]);
            }
        } else {
            T val[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i0 = base + u * 256;
                const uint32_t i = i0 < stage_total ? i0 : 0;
                const int hh = int(fdiv(i, a.fd_tw));
                const int h = hlo + hh;
                const int hc = min(max(h, 0), a.H - 1);
                val[u] = xn[int64_t(hc) * a.WL + (int(i) - hh * a.WL)];
                if (h < 0 || h >= a.H) val[u] = T(0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t i = base + u * 256;
                if (i < stage_total) tile[i] = val[u];
            }
        }
    }
    __syncthreads();
    const int RC = a.R * a.C;
    const uint32_t out_total = uint32_t(a.G) * a.fd_row.d;
    for (uint32_t v = threadIdx.x; v < out_total; v += 256) {
        int pp, col, s, tv;
        band_vector<COL>(a, v, pp, col, s, tv);
        const int p = p0 + pp;
        if (p >= a.P) continue;
        const int wcol = COL ? col * a.sw - a.pw + s * a.dw : col - a.pw;
        const int t0 = tv * VEC;
        Pack16<T> pk;
        pk.v = zero4();
        if (wcol >= 0 && wcol < a.W) {
            int r = int(fdiv(uint32_t(t0), a.fd_c));
            int c = t0 - r * a.C;
            const T* trow = tile + pp * a.sh * a.WL + wcol * a.C;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                pk.e[e] = t0 + e < RC ? trow[r * a.dh * a.WL + c] : T(0);
                if (++c == a.C) {
                    c = 0;
                    ++r;
                }
            }
        }
        T* out = static_cast<T*>(a.out) +
                 (COL ? ((int64_t(n) * a.P + p) * a.Q + col) * a.Kl + (s * a.RCp + t0)
                      : ((int64_t(n) * a.P + p) * a.W_used + col) * a.RCp + t0);
        store16(out, pk.v);
    }
}

// ---------------------------------------------------------------------------
// Generic element-wise lowering for shapes whose NCHW staging tile would not
// fit in LDS: one thread per 16-byte output vector, elements gathered one by one.
template <typename T, bool NHWC, bool COL>
__global__ void __launch_bounds__(256) lower_generic_kernel(LowerArgs a, uint32_t total_vec) {
    constexpr int VEC = Vec<T>::n;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const uint32_t cpv = a.RCp / VEC;
    for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v < total_vec; v += gridDim.x * 256u) {
        int n, p, wcol;
        int t0;
        if (COL) {
            const uint32_t vpr = a.Kl / VEC;
            const uint32_t m = v / vpr, kv = v - (v / vpr) * vpr;
            const uint32_t s = kv / cpv;
            t0 = int(kv - s * cpv) * VEC;
            const uint32_t PQ = uint32_t(a.P) * a.Q;
            n = int(m / PQ);
            const uint32_t pq = m - uint32_t(n) * PQ;
            p = int(pq / a.Q);
            const int q = int(pq - uint32_t(p) * a.Q);
            wcol = q * a.sw - a.pw + int(s) * a.dw;
        } else {
            const uint32_t vps = uint32_t(a.W_used) * cpv;
            const uint32_t strip = v / vps, rem = v - (v / vps) * vps;
            n = int(strip / a.P);
            p = int(strip - uint32_t(n) * a.P);
            const int j = int(rem / cpv);
            t0 = int(rem - uint32_t(j) * cpv) * VEC;
            wcol = j - a.pw;
        }
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int t = t0 + e;
            T val = T(0);
            if (t < a.R * a.C) {
                const int r = t / a.C, c = t - (t / a.C) * a.C;
                val = x_at<T, NHWC>(a, x, n, c, p * a.sh - a.ph + r * a.dh, wcol);
            }
            pk.e[e] = val;
        }
        store16(static_cast<T*>(a.out) + int64_t(v) * VEC, pk.v);
    }
}

// ---------------------------------------------------------------------------
// im2win and im2col with unpadded window rows (RCp == R*C, not a whole number
// of vectors; fp32 3-channel layers): the lowered buffer is a flat array of
// `elems` elements, each thread decoding VEC consecutive ones and storing them
// as one 16-byte vector (the buffer starts 16-byte aligned; the last vector
// may be partial).  Decode: fd_row divides by the elements per strip (im2win,
// W_used*R*C) or per row (im2col, S*R*C), fd_cpv by R*C.
template <typename T, bool NHWC, bool COL>
__global__ void __launch_bounds__(256) lower_unpadded_kernel(LowerArgs a, uint32_t total_vec, uint32_t elems) {
    constexpr int VEC = Vec<T>::n;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    T* __restrict__ out = static_cast<T*>(a.out);
    for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v < total_vec; v += gridDim.x * 256u) {
        const uint32_t f0 = v * VEC;
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const uint32_t f = f0 + e;
            T val = T(0);
            if (f < elems) {
                const uint32_t row = fdiv(f, a.fd_row);
                const uint32_t rem = f - row * a.fd_row.d;
                const uint32_t seg = fdiv(rem, a.fd_cpv);   // strip column j (im2win) or tap s (im2col)
                const int t = int(rem - seg * a.fd_cpv.d);
                const int r = int(fdiv(uint32_t(t), a.fd_c));
                const int c = t - r * a.C;
                int n, p, wcol;
                if (COL) {
                    const uint32_t np = fdiv(row, a.fd_q);
                    const int q = int(row - np * a.fd_q.d);
                    n = int(fdiv(np, a.fd_p));
                    p = int(np) - n * a.P;
                    wcol = q * a.sw - a.pw + int(seg) * a.dw;
                } else {
                    n = int(fdiv(row, a.fd_p));
                    p = int(row) - n * a.P;
                    wcol = int(seg) - a.pw;
                }
                val = x_at<T, NHWC>(a, x, n, c, p * a.sh - a.ph + r * a.dh, wcol);
            }
            pk.e[e] = val;
        }
        if (f0 + VEC <= elems) {
            store16(out + f0, pk.v);
        } else {
#pragma unroll
            for (int e = 0; e < VEC; ++e)
                if (f0 + e < elems) out[f0 + e] = pk.e[e];
        }
    }
}

// ---------------------------------------------------------------------------
// Filter pack: Bp[k][s*RCp + r*C + c] = w[k, c, r, s] (zeros in the padding),
// the filter matrix reshaped to the lowered row order.
struct PackArgs {
    const void* w;
    void* out;
    int32_t K, C, R, S, RCp, Kl;
    // ConvLSTM gate filters (K = 4*lstm_kh, gate order i f g o): packed row
    // hb*64 + gate*16 + l holds filter row gate*lstm_kh + hb*16 + l, so that a
    // 64-row tile carries all four gates of 16 hidden channels.  0: rows in
    // order.
    int32_t lstm_kh;
};

template <typename T, bool NHWC>
__global__ void __launch_bounds__(256) pack_filter_kernel(PackArgs a) {
    const T* __restrict__ w = static_cast<const T*>(a.w);
    T* out = static_cast<T*>(a.out);
    const int total = a.K * a.Kl;
    for (int i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
        const int kp = i / a.Kl, kk = i - (i / a.Kl) * a.Kl;
        const int k = a.lstm_kh ? ((kp % 64) / 16) * a.lstm_kh + (kp / 64) * 16 + kp % 16 : kp;
        const int s = kk / a.RCp, t = kk - (kk / a.RCp) * a.RCp;
        T val = T(0);
        if (t < a.R * a.C) {
            const int r = t / a.C, c = t - (t / a.C) * a.C;
            const int64_t src = NHWC ? ((int64_t(k) * a.R + r) * a.S + s) * a.C + c
                                     : ((int64_t(k) * a.C + c) * a.R + r) * a.S + s;
            val = w[src];
        }
        out[i] = val;
    }
}

// Filter in MFMA fragment order: Bf[nb][kk][lane][8] =
// w[nb*32 + lane%32][kk*16 + (lane/32)*8 + e] (KRSC rows, contraction index
// (r*S + s)*C + c), zero for output channels >= K.  One 16-byte chunk per
// thread.
struct FragPackArgs {
    const void* w;
    void* out;
    int32_t K, Kg, NB;   // NB = ceil(K/32)
};

template <typename T>
__global__ void __launch_bounds__(256) pack_filter_frag_kernel(FragPackArgs a) {
    const int KK = a.Kg / 16;
    const int64_t total = int64_t(a.NB) * KK * 64;
    const T* __restrict__ w = static_cast<const T*>(a.w);
    T* __restrict__ out = static_cast<T*>(a.out);
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
        const int lane = int(i & 63);
        const int64_t blk = i >> 6;
        const int kk = int(blk % KK);
        const int nb = int(blk / KK);
        const int n = nb * 32 + (lane & 31);
        u32x4 v = zero4();
        if (n < a.K) v = load16(w + int64_t(n) * a.Kg + kk * 16 + (lane >> 5) * 8);
        store16(out + i * 8, v);
    }
}

// Filter in 16x16x32 MFMA A-fragment order (the 16x16 unrolled-tap strip
// kernel): Af[nb][kk][lane][8] = w[nb*16 + lane%16][kk*32 + (lane/16)*8 + e]
// (KRSC rows, contraction index (r*S + s)*C + c), zero for output channels
// >= K.  One 16-byte chunk per thread; NB = ceil(K/16), Kg % 32 == 0.
template <typename T>
__global__ void __launch_bounds__(256) pack_filter_frag16_kernel(FragPackArgs a) {
    const int KK = a.Kg / 32;
    const int64_t total = int64_t(a.NB) * KK * 64;
    const T* __restrict__ w = static_cast<const T*>(a.w);
    T* __restrict__ out = static_cast<T*>(a.out);
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
        const int lane = int(i & 63);
        const int64_t blk = i >> 6;
        const int kk = int(blk % KK);
        const int nb = int(blk / KK);
        const int n = nb * 16 + (lane & 15);
        u32x4 v = zero4();
        if (n < a.K) v = load16(w + int64_t(n) * a.Kg + kk * 32 + (lane >> 4) * 8);
        store16(out + i * 8, v);
    }
}

// fp32 KCRS filter in the MFMA fragment order of the fp32 NCHW strip
// kernel: contraction index k' = (r*C + c)*S + s (filter row outermost), and
// Bf[nb][kk][lane][4] = w[nb*16 + lane%16][k' = kk*16 + 4*(lane/16) + e],
// zero for output channels >= K.  One 16-byte chunk per thread.
struct FragPackF32Args {
    const void* w;
    void* out;
    int32_t K, C, R, S, NB;   // NB = ceil(K/16)
};

// fp32 KCRS filter into 16x16x4 MFMA B fragments in the order of the fp32
// NCHW strip kernel: fragment kk = (cb*R + r)*S + s is the 16-deep step
// of tap (r, s) over channels cb*16 .. cb*16+15; lane (gq, l16) element e
// holds w[nb*16 + l16][cb*16 + 4*gq + e][r][s] (zero past K), at
// ((nb*KK + kk)*64 + lane)*16 bytes.  C % 16 == 0.
__global__ void __launch_bounds__(256) pack_filter_frag_f32_kernel(FragPackF32Args a) {
    const int CBN = a.C / 16;
    const int KK = CBN * a.R * a.S;
    const int64_t total = int64_t(a.NB) * KK * 64;
    const float* __restrict__ w = static_cast<const float*>(a.w);
    float* __restrict__ out = static_cast<float*>(a.out);
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
        const int lane = int(i & 63);
        const int64_t blk = i >> 6;
        const int kk = int(blk % KK);
        const int nb = int(blk / KK);
        const int n = nb * 16 + (lane & 15);
        const int strip = kk / a.S, s = kk - strip * a.S;
        const int cb = strip / a.R, r = strip - cb * a.R;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (n < a.K) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int c = cb * 16 + 4 * (lane >> 4) + e;
                v[e] = w[((int64_t(n) * a.C + c) * a.R + r) * a.S + s];
            }
        }
        store16(out + i * 4, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                                   __float_as_uint(v[3])});
    }
}

// 16-bit KRSC filter in the A-fragment order of the NHWC small-window
// kernel: fragment (hc, jb, st) (channel part hc < split, block jb < tn) of
// lane l = (g, i) (g = l/16, i = l%16) holds the 8 contraction elements of
// chunk j = st*4 + g for output channel hc*16*tn + tile16_channel(i, jb,
// tn): filter row r = j / cpr, elements t = 8*(j % cpr)
// + e of that row's run, which are w[ch][r][(t - lead) / C][(t - lead) % C]
// where 0 <= t - lead < S*C and zero elsewhere (also past R rows and past K
// channels).  One 16-byte fragment per thread.
struct Tile16PackArgs {
    const void* w;
    void* out;
    int32_t K, C, R, S, pw, ks, tn, split;
};

template <typename T>
__global__ void __launch_bounds__(256) pack_filter_tile16_kernel(Tile16PackArgs a) {
    const Tile16Geom geo = tile16_geom(a.C, a.S, a.pw);
    const int run = a.S * a.C;
    const int total = a.split * a.tn * a.ks * 64;
    const T* __restrict__ w = static_cast<const T*>(a.w);
    for (int i = int(blockIdx.x) * 256 + threadIdx.x; i < total; i += int(gridDim.x) * 256) {
        const int lane = i & 63, blk = i >> 6;
        const int st = blk % a.ks, jbg = blk / a.ks, hc = jbg / a.tn, jb = jbg - hc * a.tn;
        const int ch = hc * 16 * a.tn + tile16_channel(lane & 15, jb, a.tn);
        const int j = st * 4 + (lane >> 4);
        const int r = j / geo.cpr, t0 = (j - r * geo.cpr) * 8;
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int t = t0 + e - geo.lead;
            pk.e[e] = (ch < a.K && r < a.R && t >= 0 && t < run) ? w[(int64_t(ch) * a.R + r) * run + t]
                                                                 : from_f32<T>(0.f);
        }
        store16(static_cast<char*>(a.out) + int64_t(i) * 16, pk.v);
    }
}

}  // namespace convlower
