// Unrolled-tap strip kernel on 16x16x32 MFMAs (16-bit NHWC, unit horizontal
// dilation, S a template value).
//
// The contraction of conv_strip_rb2_kernel -- per filter row r and block of
// 32 channels, the input rows under the tile's output rows copied once into
// LDS and read by all S taps ("Enabling Memory-efficient Im2win Convolution
// with Multi-precision Support on GPU CUDA and Tensor Cores", abstract), the
// filter streamed into registers from a fragment-order copy -- with
// v_mfma_f32_16x16x32_{f16,bf16} in place of the 32x32x16 instruction.  The
// two do the same work per cycle at a given clock, but under sustained load
// the chip holds a higher shader clock for the 16x16 form (measured by the
// library's peak microbenchmarks: about 2.2 against 1.8 GHz).  One MFMA now
// covers a whole 32-channel tap step of 16 pixels and 16 output channels:
//   - strip rows keep rb2's 80 bytes; the 16 pixels of a fragment are dealt
//     to lanes as pixel 2*(l%8) + l/8 of lane l%16, so the 16 lanes the LDS
//     serves together (8 pixels two apart, two neighbouring chunks) fall in
//     16 different 4-bank groups for consecutive pixels, and a lane's A
//     address for tap s is a fixed register plus s*80 (an instruction
//     offset);
//   - the taps of a strip are one unrolled body and the filter register ring
//     is indexed at compile time (one body per ring phase), as in the 32x32
//     form;
//   - every step issues the same loads whatever the strip (past the last
//     strip they read zeros into a buffer nobody reads again), so the
//     compiler's vmcnt waits for the filter registers are exact.
#pragma once

#include "igemm_strip_rb2.hpp"

namespace convlower {

// Strip rows of 80 bytes (rb2's layout): the loads' offsets with the
// out-of-range bit ORed in where the row falls outside the image or the
// strip is past the last (valid offsets are below 2^31), no branch.
template <typename T, int NT, int STRIP>
struct PaddedStripOr : PaddedStripSrc<T, NT, STRIP> {
    __device__ __forceinline__ uint32_t voff(const GemmArgs& g, int j, int r, int cb, bool on) const {
        const int32_t h = this->hrow[j] + r * g.dh;
        const int32_t o = this->base[j] + ((r * g.dh * g.W) * g.C + cb * 32) * int32_t(sizeof(T));
        const uint32_t bad = (unsigned(h) < unsigned(g.H) ? 0u : kOutOfRange) | (on ? 0u : kOutOfRange);
        return uint32_t(o) | bad;
    }
};

// DB_MAX: how many steps ahead the filter fragments are loaded, at most
// (S - 1 for narrow filters).
template <typename T, int BM, int BN, int WGM, int WGN, int STRIP, int S, int DB_MAX>
__global__ void __launch_bounds__(64 * WGM * WGN, (strip_rb_min_blocks<BM, BN, WGM, WGN>()))
    conv_strip_rb3_kernel(GemmArgs g) {
    constexpr int DB = DB_MAX < S ? DB_MAX : S - 1;
    constexpr int NT = 64 * WGM * WGN;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int NM = TM * TN;
    constexpr int NR = DB + 1;            // filter register ring
    constexpr int BUF = STRIP * 16;       // bytes per strip buffer
    using ASrc = PaddedStripOr<T, NT, STRIP>;
    constexpr int NLA = ASrc::NL;
    constexpr int DSTEPS = S > 3 ? 3 : S - 1;                   // steps the next strip's loads are spread over
    constexpr int PER = (NLA + DSTEPS - 1) / DSTEPS;             // strip loads per such step
    // At the start of a strip's last step, before its own loads: the loads
    // issued after this wave's last load of the next strip (at step
    // DSTEPS-1, after that step's filter loads) are the filter loads of
    // steps DSTEPS .. S-2.
    constexpr int WAIT = TN * (S - 1 - DSTEPS);
    static_assert(sizeof(T) == 2, "16-bit storage");
    static_assert(STRIP % NT == 0 && WM % 16 == 0 && WN % 16 == 0, "tile shape");
    static_assert(DB >= 1 && DB < S && DSTEPS >= 1 && DSTEPS < S, "prefetch distances");
    static_assert(TN >= 2 && TN + PER <= TM * (TN - 1), "one memory operation per MFMA");
    static_assert(WAIT < 64 && NLA + NR * TN < 64, "vmcnt range");
    static_assert(S * kStripRb2RowBytes < 65536, "tap offsets fit an instruction offset");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * BUF];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile = int(xcd_tile(blockIdx.x, gridDim.x));
    const int tile_m = tile / g.tiles_n;
    const int tile_n = tile - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    const int32_t w_used = (g.Q - 1) * g.sw + (S - 1) + 1;
    const int64_t m_last = (m0 + BM < g.M ? m0 + BM : g.M) - 1;
    const int32_t g0 = int32_t(m0 / g.Q);
    const int32_t t_rows = int32_t(m_last / g.Q) - g0 + 1;

    ASrc la;
    la.init(g, g0, t_rows, w_used, tid);

    // B fragment i (16 pixels): lane (chunk c = lane/16, l = lane%16) reads
    // 16 bytes of chunk c of the strip row of pixel pl = 2*(l%8) + l/8 of
    // the fragment.  The 16 lanes the LDS serves together (lane bits 3 and 5
    // fixed) then read 8 pixels two apart in two neighbouring chunks: for
    // consecutive pixels, rows 2 apart of 80 bytes, 16 different 4-bank
    // groups.  The MFMA's B columns and output columns follow the same order.
    const int pl = 2 * (lane & 7) + ((lane >> 3) & 1);
    uint32_t aoff[TM];   // byte offset in a strip buffer at tap 0
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 16 + pl;
        int32_t sr = 0;
        if (m < g.M) {
            const int32_t gr = int32_t(m / g.Q);
            sr = (gr - g0) * w_used + (int32_t(m) - gr * g.Q) * g.sw;
        }
        aoff[i] = uint32_t(sr * kStripRb2RowBytes + (lane >> 4) * 16);
    }

    // Packed filter (pack_filter_frag16_kernel): fragment (nb, kk) at
    // ((nb*KK + kk)*64 + lane)*16 bytes, kk the 32-deep step; tap s of strip
    // (r, cb) is kk = (r*S + s)*(C/32) + cb.  (Reading the KRSC rows as they
    // are -- 16 rows of 64 bytes per fragment instead of 1 KiB in a row --
    // measured 1.3 to 1.7 times slower on the kernel-size layers.)
    const int KK = g.Kc / 32;
    const int NBt = (g.K + 15) / 16;
    const __amdgpu_buffer_rsrc_t brsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.b), 0, int(int64_t(NBt) * KK * 1024), 0x00020000);
    // Fragment j of the wave's output-channel blocks: the lane's offset in
    // the wave's first block plus a uniform j*KK KiB.  The uniform part of a
    // buffer offset is not range-checked, so blocks past the copy's last
    // (output channels past K, whose results are never stored) read the last
    // block again instead: every read stays inside the copy.
    const int nbw = min((n0 + wn * WN) / 16, NBt - 1);
    const uint32_t bfrag0 = uint32_t((int64_t(nbw) * KK * 64 + lane) * 16);
    const int bstep = KK * 1024;
    auto boff = [&](int j) { return (min(nbw + j, NBt - 1) - nbw) * bstep; };
    const int tap_bytes = g.C * 32;                                          // one tap of the filter rows
    auto kbase = [&](int r, int cb) { return (r * S * g.C + cb * 32) * 32; };   // tap 0 of strip (r, cb)

    const uint32_t lds0 = lds_offset(smem);
    auto strip_load = [&](int buf, int j, int r, int cb, bool on) __attribute__((always_inline)) {
        dma16(la.rsrc, la.voff(g, j, r, cb, on), lds0 + uint32_t(buf * BUF) + uint32_t((j * NT + wave * 64) * 16));
    };
    auto lds16 = [&](uint32_t byte_off) __attribute__((always_inline)) { return load16(smem + byte_off); };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int CB = g.C / 32;
    const int nstrips = g.R * CB;

    // Prologue: strip 0 into buffer 0, the filter fragments of taps 0 .. DB-1
    // of strip 0, then the A fragments of its first step.
#pragma unroll
    for (int j = 0; j < NLA; ++j) strip_load(0, j, 0, 0, true);
    u32x4 fb[NR][TN];
    static_for<DB>([&](auto dc) __attribute__((always_inline)) {
        constexpr int d = decltype(dc)::value;
#pragma unroll
        for (int j = 0; j < TN; ++j) fb[d][j] = buffer_load16(brsrc, bfrag0, d * tap_bytes + boff(j));
    });
    wait_vmcnt<0>();
    lds_barrier();
    u32x4 fa[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = lds16(aoff[i]);

    // One strip: S steps.  Ring phase PH: the filter fragments of tap s are
    // in set (PH + s) % NR.
    auto strip = [&](auto phc, int r, int cb, int r1, int cb1, int buf, bool has_next) __attribute__((always_inline)) {
        constexpr int PH = decltype(phc)::value;
        const int kb = kbase(r, cb);
        const int kb1 = has_next ? kbase(r1, cb1) : 0;
        uint32_t abase[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) abase[i] = aoff[i] + uint32_t(buf * BUF);
        static_for<S>([&](auto sc) __attribute__((always_inline)) {
            constexpr int s = decltype(sc)::value;
            constexpr int RC = (PH + s) % NR;
            constexpr int RL = (PH + s + DB) % NR;
            // filter fragments of tap s + DB: this strip or the next; past
            // the last strip, position 0 again into a set nobody reads
            constexpr bool nxt = s + DB >= S;
            constexpr int sb = nxt ? s + DB - S : s + DB;
            const int kbb = nxt ? (has_next ? kb1 + sb * tap_bytes : 0) : kb + sb * tap_bytes;
            if constexpr (s == S - 1) {
                // the next strip landed for this wave, then for every wave;
                // every wave's reads of this strip are done
                wait_vmcnt<WAIT>();
                __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
                lds_barrier();
            }
            // MFMAs fragment by fragment (i outer): once fragment i's last
            // MFMA has issued, its register takes the next step's fragment i
            // (tap s+1, or tap 0 of the next strip), which is first needed
            // NM - TN MFMAs later.  Between them, the filter loads of step
            // k+DB and, in the first DSTEPS steps, the next strip's loads.
            static_for<NM>([&](auto idxc) __attribute__((always_inline)) {
                constexpr int idx = decltype(idxc)::value;
                constexpr int i = idx / TN, j = idx % TN;
                acc[i][j] = Mfma<T>::run(fb[RC][j], fa[i], acc[i][j]);
                if constexpr (j == TN - 1) {
                    if constexpr (s + 1 < S)
                        fa[i] = lds16(abase[i] + uint32_t((s + 1) * kStripRb2RowBytes));
                    else
                        fa[i] = lds16(aoff[i] + uint32_t((buf ^ 1) * BUF));
                } else if constexpr (idx % TN < TN - 1 && idx / TN * (TN - 1) + idx % TN < TN) {
                    constexpr int q = idx / TN * (TN - 1) + idx % TN;   // q-th MFMA without an LDS read
                    fb[RL][q] = buffer_load16(brsrc, bfrag0, kbb + boff(q));
                } else if constexpr (s < DSTEPS) {
                    constexpr int q = idx / TN * (TN - 1) + idx % TN - TN;
                    if constexpr (q >= 0 && q < PER && s * PER + q < NLA)
                        strip_load(buf ^ 1, s * PER + q, r1, cb1, has_next);
                }
                __builtin_amdgcn_sched_barrier(0);
            });
        });
    };

    int r = 0, cb = 0, ph = 0;
    for (int j = 0; j < nstrips; ++j) {
        int r1 = r, cb1 = cb + 1;
        if (cb1 == CB) {
            cb1 = 0;
            ++r1;
        }
        const bool has_next = j + 1 < nstrips;
        const int buf = j & 1;
        static_for<NR>([&](auto pc) __attribute__((always_inline)) {
            if (ph == decltype(pc)::value) strip(pc, r, cb, r1, cb1, buf, has_next);
        });
        ph = (ph + S) % NR;
        r = r1;
        cb = cb1;
    }
    // strip loads past the last strip still write this workgroup's LDS
    wait_vmcnt<0>();

    // Fused epilogue: lane (c = lane/16) of fragment (i, j) holds output
    // channels j*16 + 4c .. +3 of its pixel pl.
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    const int kl = 4 * (lane >> 4);
    float bv[TN][4];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int k = n0 + wn * WN + j * 16 + kl;
        if (bias && (g.K & 3) == 0 && k + 3 < g.K) {
            union {
                u32x2 u;
                T e[4];
            } pk;
            pk.u = *reinterpret_cast<const u32x2*>(bias + k);
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[j][e] = to_f32(pk.e[e]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[j][e] = (bias && k + e < g.K) ? to_f32(bias[k + e]) : 0.f;
        }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int64_t m = m0 + wm * WM + i * 16 + pl;
        if (m >= g.M) continue;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int k = n0 + wn * WN + j * 16 + kl;
            T* dst = y + m * g.K + k;
            if (k + 3 < g.K && (g.K & 3) == 0) {
                union {
                    u32x2 u;
                    T e[4];
                } pk;
#pragma unroll
                for (int e = 0; e < 4; ++e) pk.e[e] = from_f32<T>(acc[i][j][e] + bv[j][e]);
                *reinterpret_cast<u32x2*>(dst) = pk.u;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (k + e < g.K) dst[e] = from_f32<T>(acc[i][j][e] + bv[j][e]);
            }
        }
    }
}

}  // namespace convlower
