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
    int32_t chunk;    // strip columns (im2win NCHW) or output columns (im2col NCHW) per block
    int32_t lds_ld;   // LDS row pitch (elements) of the NCHW staging tile
    // NCHW input split over two tensors (a ConvLSTM step's x and h): channels
    // c < C1 come from x (C1 per image), the rest from x2 (C - C1 per image).
    // C1 == C and x2 == nullptr for an ordinary convolution.
    const void* x2;
    int32_t C1;
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
// im2win, NHWC input: one thread per 16-byte vector of the strip.  When C is a
// whole number of vectors, a vector of the strip is a vector of one x row, so
// the copy is 16-byte load -> 16-byte store; otherwise it gathers elements.
// grid.x = N*P strips, grid.y = ceil(W_used*RCp/VEC / 256).
template <typename T, bool C_VEC>
__global__ void __launch_bounds__(256) im2win_nhwc_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    const int strip = blockIdx.x;
    const int cpv = a.RCp / VEC;                 // vectors per strip column
    const int v = blockIdx.y * 256 + threadIdx.x;
    if (v >= a.W_used * cpv) return;
    const int n = strip / a.P, p = strip - (strip / a.P) * a.P;
    const int j = v / cpv;
    const int t0 = (v - j * cpv) * VEC;
    const int wcol = j - a.pw;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    T* out = static_cast<T*>(a.out) + (int64_t(strip) * a.W_used * a.RCp + int64_t(v) * VEC);
    if (C_VEC) {
        const int r = t0 / a.C, c0 = t0 - (t0 / a.C) * a.C;
        const int h = p * a.sh - a.ph + r * a.dh;
        u32x4 val = zero4();
        if (h >= 0 && h < a.H && wcol >= 0 && wcol < a.W)
            val = load16(x + ((int64_t(n) * a.H + h) * a.W + wcol) * a.C + c0);
        store16(out, val);
    } else {
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int t = t0 + e;
            T val = T(0);
            if (t < a.R * a.C) {
                const int r = t / a.C, c = t - (t / a.C) * a.C;
                val = x_at<T, true>(a, x, n, c, p * a.sh - a.ph + r * a.dh, wcol);
            }
            pk.e[e] = val;
        }
        store16(out, pk.v);
    }
}

// ---------------------------------------------------------------------------
// NCHW input: x rows are contiguous along w, the strip is contiguous along
// (r, c) inside a column, so stage through LDS: read coalesced along w into a
// [column][r*C + c] tile, then write whole 16-byte strip vectors.
// Tile rows [j0, j0 + ncols) of strip (n, p); LDS pitch a.lds_ld elements.
template <typename T>
__device__ __forceinline__ void stage_strip_nchw(const LowerArgs& a, T* tile, int n, int p, int j0, int ncols) {
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const int RC = a.R * a.C;
    const int total = ncols * RC;
    for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
        const int jj = idx % ncols;
        const int rc = idx / ncols;
        const int c = rc % a.C, r = rc / a.C;
        const int h = p * a.sh - a.ph + r * a.dh;
        tile[jj * a.lds_ld + rc] = x_at<T, false>(a, x, n, c, h, j0 + jj - a.pw);
    }
}

// grid.x = N*P strips, grid.y = ceil(W_used / chunk); dynamic LDS = chunk*lds_ld elements.
template <typename T>
__global__ void __launch_bounds__(256) im2win_nchw_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* tile = reinterpret_cast<T*>(lds_raw);
    const int strip = blockIdx.x;
    const int n = strip / a.P, p = strip - (strip / a.P) * a.P;
    const int j0 = blockIdx.y * a.chunk;
    const int ncols = min(a.chunk, a.W_used - j0);
    stage_strip_nchw<T>(a, tile, n, p, j0, ncols);
    __syncthreads();
    const int RC = a.R * a.C;
    const int cpv = a.RCp / VEC;
    T* out = static_cast<T*>(a.out) + (int64_t(strip) * a.W_used + j0) * a.RCp;
    for (int idx = threadIdx.x; idx < ncols * cpv; idx += blockDim.x) {
        const int jj = idx / cpv, tv = idx - (idx / cpv) * cpv;
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int t = tv * VEC + e;
            pk.e[e] = t < RC ? tile[jj * a.lds_ld + t] : T(0);
        }
        store16(out + int64_t(jj) * a.RCp + tv * VEC, pk.v);
    }
}

// ---------------------------------------------------------------------------
// im2col, NHWC input: one thread per 16-byte vector of Col; grid-stride over
// M*Kl/VEC vectors (checked on the host to fit 32 bits).
template <typename T, bool C_VEC>
__global__ void __launch_bounds__(256) im2col_nhwc_kernel(LowerArgs a, uint32_t total_vec) {
    constexpr int VEC = Vec<T>::n;
    const T* __restrict__ x = static_cast<const T*>(a.x);
    const uint32_t vpr = a.Kl / VEC;   // vectors per Col row
    const uint32_t cpv = a.RCp / VEC;
    const uint32_t PQ = uint32_t(a.P) * a.Q;
    for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v < total_vec; v += gridDim.x * 256u) {
        const uint32_t m = v / vpr, kv = v - (v / vpr) * vpr;
        const uint32_t s = kv / cpv;
        const int t0 = int(kv - s * cpv) * VEC;
        const uint32_t n = m / PQ, pq = m - (m / PQ) * PQ;
        const int p = int(pq / a.Q), q = int(pq - (pq / a.Q) * a.Q);
        const int wcol = q * a.sw - a.pw + int(s) * a.dw;
        T* out = static_cast<T*>(a.out) + int64_t(v) * VEC;
        if (C_VEC) {
            const int r = t0 / a.C, c0 = t0 - (t0 / a.C) * a.C;
            const int h = p * a.sh - a.ph + r * a.dh;
            u32x4 val = zero4();
            if (h >= 0 && h < a.H && wcol >= 0 && wcol < a.W)
                val = load16(x + ((int64_t(n) * a.H + h) * a.W + wcol) * a.C + c0);
            store16(out, val);
        } else {
            Pack16<T> pk;
#pragma unroll
            for (int e = 0; e < VEC; ++e) {
                const int t = t0 + e;
                T val = T(0);
                if (t < a.R * a.C) {
                    const int r = t / a.C, c = t - (t / a.C) * a.C;
                    val = x_at<T, true>(a, x, int(n), c, p * a.sh - a.ph + r * a.dh, wcol);
                }
                pk.e[e] = val;
            }
            store16(out, pk.v);
        }
    }
}

// im2col, NCHW input: a block stages the strip columns its output columns
// [q0, q0 + chunk) need for one (n, p), then writes those Col rows.
// grid.x = N*P, grid.y = ceil(Q / chunk); dynamic LDS = cols*lds_ld elements
// with cols = (chunk-1)*sw + (S-1)*dw + 1.
template <typename T>
__global__ void __launch_bounds__(256) im2col_nchw_kernel(LowerArgs a) {
    constexpr int VEC = Vec<T>::n;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    T* tile = reinterpret_cast<T*>(lds_raw);
    const int strip = blockIdx.x;
    const int n = strip / a.P, p = strip - (strip / a.P) * a.P;
    const int q0 = blockIdx.y * a.chunk;
    const int nq = min(a.chunk, a.Q - q0);
    const int j0 = q0 * a.sw;
    const int ncols = (nq - 1) * a.sw + (a.S - 1) * a.dw + 1;
    stage_strip_nchw<T>(a, tile, n, p, j0, ncols);
    __syncthreads();
    const int RC = a.R * a.C;
    const int cpv = a.RCp / VEC;
    const int vpr = a.Kl / VEC;
    T* out = static_cast<T*>(a.out) + (int64_t(strip) * a.Q + q0) * a.Kl;
    for (int idx = threadIdx.x; idx < nq * vpr; idx += blockDim.x) {
        const int qq = idx / vpr, kv = idx - (idx / vpr) * vpr;
        const int s = kv / cpv, tv = kv - (kv / cpv) * cpv;
        const int jj = qq * a.sw + s * a.dw;
        Pack16<T> pk;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            const int t = tv * VEC + e;
            pk.e[e] = t < RC ? tile[jj * a.lds_ld + t] : T(0);
        }
        store16(out + int64_t(qq) * a.Kl + kv * VEC, pk.v);
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
