// Strip-staged implicit contraction (16-bit NHWC, C a multiple of 32): the
// im2win window layout built in LDS instead of in a workspace.
//
// "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
// on GPU CUDA and Tensor Cores" (abstract): the im2win transformation keeps
// one copy of each input row under a row of output pixels, and every kernel
// tap reads its window as a contiguous run of that copy.  Here the copy lives
// only in LDS: for filter row r and a block of 32 channels the workgroup
// copies, once, the input rows h = p*sh - ph + r*dh under the output rows
// (n, p) its pixel tile touches -- W_used = (Q-1)*sw + (S-1)*dw + 1 columns
// each, zero outside the image -- and then serves all S taps of that filter
// row from it: the window of pixel (n, p, q) for tap s starts at strip row
// t*W_used + q*sw + s*dw (t = the output row's index within the tile).
// Compared with gathering a window tile per tap from global memory, the
// global (L2) traffic for the A side drops by about a factor S.
//
// Contraction order: steps (r, cb, s), s fastest; one step is 32 channels of
// one tap, i.e. a 32-deep slice of the filter rows w[k][r][s][cb*32 ..].
//
// Schedule (one wave per SIMD, 32 x 32 x 16 MFMAs, register tiles as in
// conv_gemm_wide_kernel): strips are double-buffered, filter tiles run in a
// ring of BST stages.  At the boundary of step k (its second 16-deep half):
//   wait until the filter tile of step k+1 (and its strip, when step k+1
//   starts one) has landed -> barrier -> read the fragments of step k+1 ->
//   MFMAs of step k, with the loads of the strip after next (when step k
//   starts a strip) and of the filter tile of step k+BST-1 spread between
//   them.
// The strip buffer refilled at the first step of strip j held strip j-1,
// whose last reads were consumed by the MFMAs of step k-1; the filter stage
// refilled held step k-1's tile.  Both are behind this barrier.
#pragma once

#include "igemm_wide.hpp"

namespace convlower {

// The input strip of one (r, channel block): STRIP chunk slots of 16 bytes
// (a multiple of NT), slot (row, c) at 16*(4*row + swz(row, c)).
template <typename T, int NT, int STRIP>
struct StripSrc {
    static constexpr int NL = STRIP / NT;
    int32_t base[NL];   // bytes to x[n][p*sh - ph][w][chunk*8] (r = 0, block 0)
    int32_t hrow[NL];   // p*sh - ph, or far out of range for slots past the strip / image columns
    i32x4 rsrc;

    __device__ __forceinline__ void init(const GemmArgs& g, int32_t g0, int32_t t_rows, int32_t w_used, int tid) {
        const int64_t x_bytes = (g.M / g.PQ) * int64_t(g.H) * g.W * g.C * int64_t(sizeof(T));
        rsrc = make_rsrc(g.a, uint32_t(x_bytes < int64_t(0x7fffffff) ? x_bytes : int64_t(0x7fffffff)));
        const int32_t P = g.PQ / g.Q;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int slot = j * NT + tid;
            const int sr = slot >> 2;
            const int chunk = swz_chunk<4, 1>(sr, slot & 3);
            const int t = sr / w_used;
            const int col = sr - t * w_used;
            const int32_t gr = g0 + (t < t_rows ? t : 0);
            const int32_t n = gr / P;
            const int32_t p = gr - n * P;
            const int32_t w = col - g.pw;
            const int32_t hv = p * g.sh - g.ph;
            const bool ok = t < t_rows && unsigned(w) < unsigned(g.W);
            base[j] = ((n * g.H + hv) * g.W + w) * g.C * int32_t(sizeof(T)) + chunk * 16;
            hrow[j] = ok ? hv : -(1 << 28);
        }
    }
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j, int r, int cb) const {
        const int32_t h = hrow[j] + r * g.dh;
        const int32_t o = base[j] + ((r * g.dh * g.W) * g.C + cb * 32) * int32_t(sizeof(T));
        return unsigned(h) < unsigned(g.H) ? uint32_t(o) : kOutOfRange;
    }
};

// Filter rows n0 .. n0+BN-1 of w[K][Kg], 32 elements at contraction position
// `pos` per step (row chunks swizzled like the strip).
template <typename T, int BN, int NT>
struct FilterRowsAt {
    static constexpr int CHUNKS = BN * 4;
    static constexpr int NL = (CHUNKS + NT - 1) / NT;
    static_assert(CHUNKS % NT == 0 || CHUNKS < NT, "whole wave loads");
    uint32_t roff[NL];
    bool ok[NL];
    i32x4 rsrc;

    __device__ __forceinline__ void init(const GemmArgs& g, int n0, int tid) {
        const int64_t rows = g.K - n0 < BN ? g.K - n0 : BN;
        const T* base = static_cast<const T*>(g.b) + int64_t(n0) * g.ldb;
        const int64_t bytes = rows * g.ldb * int64_t(sizeof(T));
        rsrc = make_rsrc(base, uint32_t(bytes < int64_t(0x7fffffff) ? bytes : int64_t(0x7fffffff)));
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int slot = j * NT + tid;
            const int row = slot >> 2;
            const int chunk = swz_chunk<4, 1>(row, slot & 3);
            ok[j] = row < BN && row < rows;
            roff[j] = uint32_t((int64_t(ok[j] ? row : 0) * g.ldb + chunk * 8) * int64_t(sizeof(T)));
        }
    }
    __device__ __forceinline__ uint32_t voff(int j, int pos) const {
        return ok[j] ? roff[j] + uint32_t(pos * int(sizeof(T))) : kOutOfRange;
    }
};

// Position (r, cb, s) of a step; s fastest.
struct StepPos {
    int r, cb, s;
    __device__ __forceinline__ void advance(int S, int CB) {
        if (++s == S) {
            s = 0;
            if (++cb == CB) {
                cb = 0;
                ++r;
            }
        }
    }
};

template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int BST>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) conv_strip_kernel(GemmArgs g) {
    constexpr int NT = 64 * WGM * WGN;
    constexpr int NW = WGM * WGN;
    constexpr int VEC = Vec<T>::n;
    constexpr int BK = 32;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int STRIP_ELEMS = STRIP * VEC;
    constexpr int B_ELEMS = BN * BK;
    using ASrc = StripSrc<T, NT, STRIP>;
    using BSrc = FilterRowsAt<T, BN, NT>;
    constexpr int NLA = ASrc::NL, NLB = BSrc::NL;
    constexpr int B_WAVES = BN * 4 >= NT ? NW : (BN * 4) / 64;
    static_assert(sizeof(T) == 2 && VEC == 8, "16-bit storage");
    static_assert(STRIP % NT == 0 && WM % 32 == 0 && WN % 32 == 0, "tile shape");
    static_assert(BST >= 4, "filter ring: the tile of step k+BST-1 goes into the stage of step k-1");
    static_assert(NLA + 2 * NLB < 64, "vmcnt range");

    __shared__ __attribute__((aligned(16))) T smem[2 * STRIP_ELEMS + BST * B_ELEMS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int tile_n = tile - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    // Output rows (n*P + p) under the tile, and the strip geometry.
    const int32_t w_used = (g.Q - 1) * g.sw + (g.S - 1) * g.dw + 1;
    const int64_t m_last = (m0 + BM < g.M ? m0 + BM : g.M) - 1;
    const int32_t g0 = int32_t(m0 / g.Q);
    const int32_t t_rows = int32_t(m_last / g.Q) - g0 + 1;

    ASrc la;
    BSrc lb;
    la.init(g, g0, t_rows, w_used, tid);
    lb.init(g, n0, tid);

    // Strip row of each of this lane's fragment rows, for tap s = 0.
    int32_t srow[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 32 + (lane & 31);
        int32_t sr = 0;
        if (m < g.M) {
            const int32_t gr = int32_t(m / g.Q);
            sr = (gr - g0) * w_used + (int32_t(m) - gr * g.Q) * g.sw;
        }
        srow[i] = sr;
    }

    const uint32_t lds0 = lds_offset(smem);
    const uint32_t lds_b0 = lds0 + uint32_t(2 * STRIP_ELEMS * sizeof(T));
    auto strip_load = [&](int buf, int j, int r, int cb) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, r, cb), lds0 + uint32_t(buf * STRIP_ELEMS * sizeof(T)) + uint32_t((j * NT + wave * 64) * 16));
    };
    auto b_load = [&](int st, int j, int pos) __attribute__((always_inline)) {
        if (wave < B_WAVES)
            dma16(lb.rsrc, lb.voff(j, pos), lds_b0 + uint32_t(st * B_ELEMS * sizeof(T)) + uint32_t((j * NT + wave * 64) * 16));
    };

    // Fragments of sub-step kb (16 deep) of a step whose strip sits in buffer
    // `buf`, tap s, filter tile in stage `st`.
    const int frag_row = lane & 31;
    const int frag_chunk = lane >> 5;
    auto read = [&](u32x4 (&fa)[TM], u32x4 (&fb)[TN], int buf, int s, int st, int kb) __attribute__((always_inline)) {
        const T* sa = smem + buf * STRIP_ELEMS;
        const int soff = s * g.dw;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int row = srow[i] + soff;
            fa[i] = load16(sa + (row * 4 + swz_chunk<4, 1>(row, kb * 2 + frag_chunk)) * VEC);
        }
        const T* sb = smem + 2 * STRIP_ELEMS + st * B_ELEMS;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int row = wn * WN + j * 32 + frag_row;
            fb[j] = load16(sb + (row * 4 + swz_chunk<4, 1>(row, kb * 2 + frag_chunk)) * VEC);
        }
    };

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    const int S = g.S, CB = g.C / 32;
    const int nsteps = g.R * CB * S;
    const int nstrips = g.R * CB;

    // Prologue: strip 0, filter tiles of steps 0 .. BST-2.
    StepPos pb{0, 0, 0};   // position of the next filter tile to load
#pragma unroll
    for (int j = 0; j < NLA; ++j) strip_load(0, j, 0, 0);
#pragma unroll
    for (int st = 0; st < BST - 1; ++st) {
        if (st < nsteps) {
            const int pos = (pb.r * S + pb.s) * g.C + pb.cb * 32;
#pragma unroll
            for (int j = 0; j < NLB; ++j) b_load(st, j, pos);
            pb.advance(S, CB);
        }
    }
    // strip 0 and filter tile 0 landed; tiles 1 .. BST-2 may stay in flight
    if (nsteps >= BST - 1) {
        if (wave < B_WAVES)
            wait_vmcnt<(BST - 2) * NLB>();
        else
            wait_vmcnt<0>();
    } else {
        wait_vmcnt<0>();
    }
    lds_barrier();

    u32x4 fa0[TM], fb0[TN], fa1[TM], fb1[TN];
    read(fa0, fb0, 0, 0, 0, 0);

    StepPos pc{0, 0, 0};      // step k
    int strip_k = 0;          // strip index of step k
    int stage_k = 0;          // filter stage of step k
    int next_strip = 1;       // next strip to load
    StepPos ps{0, 1, 0};      // (r, cb) of next_strip
    if (ps.cb == CB) {
        ps.cb = 0;
        ++ps.r;
    }
    bool strip_issued_prev = false;   // did the previous boundary load a strip?

    for (int k = 0; k < nsteps; ++k) {
        // ---- first 16-deep half: fragments of the second half, then MFMAs
        read(fa1, fb1, strip_k & 1, pc.s, stage_k, 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = Mfma32<T>::run(fb0[j], fa0[i], acc[i][j]);
        __builtin_amdgcn_sched_barrier(0);

        // ---- boundary: step k+1's data -> barrier -> its fragments
        StepPos pn = pc;
        pn.advance(S, CB);
        const bool last = k + 1 == nsteps;
        const bool new_strip = !last && pn.s == 0;
        // Loads issued after the filter tile of step k+1: the tiles of steps
        // k+2 .. k+BST-2, plus a strip issued at the previous boundary unless
        // step k+1 needs that very strip.
        if (k + BST - 1 <= nsteps) {
            if (wave < B_WAVES) {
                if (strip_issued_prev && !new_strip)
                    wait_vmcnt<(BST - 3) * NLB + NLA>();
                else
                    wait_vmcnt<(BST - 3) * NLB>();
            } else {
                if (strip_issued_prev && !new_strip)
                    wait_vmcnt<NLA>();
                else
                    wait_vmcnt<0>();
            }
        } else {
            wait_vmcnt<0>();
        }
        lds_barrier();
        const int strip_n = new_strip ? strip_k + 1 : strip_k;
        const int stage_n = stage_k + 1 == BST ? 0 : stage_k + 1;
        read(fa0, fb0, (last ? strip_k : strip_n) & 1, last ? pc.s : pn.s, stage_n, 0);
        __builtin_amdgcn_sched_barrier(0);

        // ---- second half: MFMAs, with this boundary's loads between them
        const bool do_strip = pc.s == 0 && next_strip < nstrips;
        const bool do_b = pb.r < g.R;
        const int st_b = stage_k == 0 ? BST - 1 : stage_k - 1;
        const int pos_b = (pb.r * S + pb.s) * g.C + pb.cb * 32;
        static_for<TM * TN>([&](auto idxc) __attribute__((always_inline)) {
            constexpr int idx = decltype(idxc)::value;
            constexpr int i = idx / TN, j = idx % TN;
            acc[i][j] = Mfma32<T>::run(fb1[j], fa1[i], acc[i][j]);
            if constexpr (idx < NLA) {
                if (do_strip) strip_load(next_strip & 1, idx, ps.r, ps.cb);
            } else if constexpr (idx < NLA + NLB) {
                if (do_b) b_load(st_b, idx - NLA, pos_b);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        static_for<(NLA + NLB > TM * TN ? NLA + NLB - TM * TN : 0)>([&](auto rc) __attribute__((always_inline)) {
            constexpr int idx = TM * TN + decltype(rc)::value;
            if constexpr (idx < NLA) {
                if (do_strip) strip_load(next_strip & 1, idx, ps.r, ps.cb);
            } else {
                if (do_b) b_load(st_b, idx - NLA, pos_b);
            }
        });
        __builtin_amdgcn_sched_barrier(0);
        if (do_strip) {
            ++next_strip;
            if (++ps.cb == CB) {
                ps.cb = 0;
                ++ps.r;
            }
        }
        if (do_b) pb.advance(S, CB);
        strip_issued_prev = do_strip;
        pc = pn;
        strip_k = strip_n;
        stage_k = stage_n;
    }

    store_tile32_nhwc<T, WM, WN, TM, TN>(g, acc, m0, n0, wm, wn, lane);
}

}  // namespace convlower
