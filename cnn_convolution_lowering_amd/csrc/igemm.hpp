// The contraction Y[M x K] = A[M x Kl] * Bp[K x Kl]^T on gfx950 MFMA, with
// the bias add, rounding and NCHW / NHWC store fused into its epilogue.
//
// "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
// Extension", section "Transforming Conv2D into im2col and GEMM": output
// matrix = filter matrix x lowered input; section "Global Memory and Shared
// Memory": reusable tiles are staged in on-chip memory and reused by the
// threads of a block.  Here a 256-thread workgroup owns a BM x BN output tile;
// its A (lowered input) and B (packed filter) tiles are staged through LDS in
// two buffers, so the 16-byte global loads of tile k+1 are in flight while
// the MFMAs consume tile k; LDS rows are padded by one 16-byte vector so the
// fragment reads of 16 consecutive rows fall in distinct banks.
//
// A row m = (n, p, q) starts at n*sN + p*sP + q*sQ and its element kk sits at
// (kk / RCp)*sS + kk % RCp past that, which covers the im2win strips
// (sQ = sw*RCp, sS = dw*RCp), explicit im2col rows (sQ = Kl, one segment) and
// a 1x1 NHWC input read in place (sQ = sw*C).
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
    const void* a;
    const void* b;
    const void* bias;   // NULL: no bias
    void* y;
    int64_t M;          // output pixels N*P*Q
    int32_t K;          // output channels
    int32_t Kl;         // lowered contraction length (multiple of VEC)
    int32_t PQ, Q;      // decode m -> (n, p, q)
    int64_t sN, sP, sQ; // A row offset (elements)
    int32_t RCp, sS;    // A column offset
    int32_t ldb;        // Bp row pitch (elements)
    int32_t tiles_n;    // ceil(K / BN)
};

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

// BM x BN output tile, BK-deep LDS stages, WGM x WGN waves (4 in all).
// NHWC_OUT: the MFMA is fed (filter, pixel) so a lane ends with 4 consecutive
// output channels of one pixel (contiguous in NPQK); otherwise (pixel, filter)
// so a lane ends with 4 consecutive pixels of one channel (contiguous in NKPQ).
template <typename T, int BM, int BN, int BK, int WGM, int WGN, bool NHWC_OUT>
__global__ void __launch_bounds__(256) igemm_kernel(GemmArgs g) {
    constexpr int VEC = Vec<T>::n;
    constexpr int KV = BK / VEC;      // 16-byte vectors per tile row
    constexpr int LDK = BK + VEC;     // LDS row pitch (elements), one vector of padding
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 16, TN = WN / 16;
    constexpr int KB = 4 * VEC;       // contraction depth of one fragment step
    constexpr int A_LD = (BM * KV + 255) / 256;
    constexpr int B_LD = (BN * KV + 255) / 256;
    static_assert(WGM * WGN == 4, "four waves per workgroup");
    static_assert(BK % KB == 0 && 256 % KV == 0, "tile depth");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile");

    __shared__ __attribute__((aligned(16))) T sA[2][BM * LDK];
    __shared__ __attribute__((aligned(16))) T sB[2][BN * LDK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WGN, wn = wave - (wave / WGN) * WGN;
    const int tile_m = blockIdx.x / g.tiles_n;
    const int tile_n = blockIdx.x - tile_m * g.tiles_n;
    const int64_t m0 = int64_t(tile_m) * BM;
    const int n0 = tile_n * BN;

    const T* __restrict__ A = static_cast<const T*>(g.a);
    const T* __restrict__ B = static_cast<const T*>(g.b);

    // Load slots: vector v = tid + i*256 of a tile is row v / KV, column
    // (v % KV)*VEC; since 256 % KV == 0 the column is the same for every slot.
    const int kv = tid % KV;
    int64_t a_off[A_LD];
    bool a_ok[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int v = tid + i * 256;
        const int row = v / KV;
        const int64_t m = m0 + row;
        a_ok[i] = (v < BM * KV) && (m < g.M);
        const int32_t mm = a_ok[i] ? int32_t(m) : 0;   // M < 2^31 (checked on the host)
        const int32_t n = mm / g.PQ;
        const int32_t pq = mm - n * g.PQ;
        const int32_t p = pq / g.Q, q = pq - (pq / g.Q) * g.Q;
        a_off[i] = int64_t(n) * g.sN + int64_t(p) * g.sP + int64_t(q) * g.sQ;
    }
    int64_t b_off[B_LD];
    bool b_ok[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int v = tid + i * 256;
        const int k = n0 + v / KV;
        b_ok[i] = (v < BN * KV) && (k < g.K);
        b_off[i] = int64_t(b_ok[i] ? k : 0) * g.ldb;
    }

    // Column state of this thread's vector: absolute lowered column kk, and
    // its split into segment offset a_seg = (kk / RCp)*sS and remainder a_t.
    int kk = kv * VEC;
    int a_t = kk % g.RCp;
    int64_t a_seg = int64_t(kk / g.RCp) * g.sS;

    u32x4 ra[A_LD], rb[B_LD];
    auto gload = [&]() {
        const bool kin = kk < g.Kl;
#pragma unroll
        for (int i = 0; i < A_LD; ++i)
            ra[i] = (a_ok[i] && kin) ? load16(A + a_off[i] + a_seg + a_t) : zero4();
#pragma unroll
        for (int i = 0; i < B_LD; ++i)
            rb[i] = (b_ok[i] && kin) ? load16(B + b_off[i] + kk) : zero4();
    };
    auto advance = [&]() {
        kk += BK;
        a_t += BK;
        while (a_t >= g.RCp) {
            a_t -= g.RCp;
            a_seg += g.sS;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_LD; ++i) {
            const int v = tid + i * 256;
            if (v < BM * KV) store16(&sA[buf][(v / KV) * LDK + kv * VEC], ra[i]);
        }
#pragma unroll
        for (int i = 0; i < B_LD; ++i) {
            const int v = tid + i * 256;
            if (v < BN * KV) store16(&sB[buf][(v / KV) * LDK + kv * VEC], rb[i]);
        }
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = (g.Kl + BK - 1) / BK;
    gload();
    sstore(0);
    __syncthreads();

    const int frag_row = lane & 15;
    const int frag_k = (lane >> 4) * VEC;
    for (int kt = 0; kt < nkt; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < nkt;
        if (more) {
            advance();
            gload();
        }
#pragma unroll
        for (int kb = 0; kb < BK / KB; ++kb) {
            u32x4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                fa[i] = load16(&sA[cur][(wm * WM + i * 16 + frag_row) * LDK + kb * KB + frag_k]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                fb[j] = load16(&sB[cur][(wn * WN + j * 16 + frag_row) * LDK + kb * KB + frag_k]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = NHWC_OUT ? Mfma<T>::run(fb[j], fa[i], acc[i][j]) : Mfma<T>::run(fa[i], fb[j], acc[i][j]);
        }
        if (more) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue: y = round(acc + bias[k]).
    const T* __restrict__ bias = static_cast<const T*>(g.bias);
    T* __restrict__ y = static_cast<T*>(g.y);
    if (NHWC_OUT) {
        // acc[i][j][e]: channel n0 + wn*WN + j*16 + 4*(lane>>4) + e, pixel m0 + wm*WM + i*16 + (lane&15)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int64_t m = m0 + wm * WM + i * 16 + (lane & 15);
            if (m >= g.M) continue;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int k = n0 + wn * WN + j * 16 + 4 * (lane >> 4);
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    v[e] = acc[i][j][e] + ((bias && k + e < g.K) ? to_f32(bias[k + e]) : 0.f);
                T* dst = y + m * g.K + k;
                if (k + 3 < g.K && (g.K & 3) == 0) {
                    if (sizeof(T) == 4) {
                        store16(dst, u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]),
                                           __float_as_uint(v[2]), __float_as_uint(v[3])});
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
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int k = n0 + wn * WN + j * 16 + (lane & 15);
            if (k >= g.K) continue;
            const float bk = bias ? to_f32(bias[k]) : 0.f;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int64_t mb = m0 + wm * WM + i * 16 + 4 * (lane >> 4);
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

}  // namespace convlower
