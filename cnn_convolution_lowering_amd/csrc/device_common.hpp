// Device-side types and helpers shared by the lowering and contraction kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace convlower {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Elements per 16-byte vector: every global load and store of the lowering
// and contraction kernels moves whole 16-byte vectors where the layout allows.
template <typename T>
struct Vec {
    static constexpr int n = 16 / sizeof(T);
};

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ __forceinline__ void store16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Unsigned division by a divisor fixed at launch, as multiply-high, add and
// shift: the round-up multiplier of Granlund and Montgomery, "Division by
// Invariant Integers using Multiplication" (PLDI 1994), section 4.  With
// l = ceil(log2 d) and m = floor(2^32 * (2^l - d) / d) + 1, floor(n / d) =
// (mulhi(m, n) + n) >> l for every n < 2^32; the sum is formed in 32 bits,
// which is exact while n < 2^31 (mulhi(m, n) < n).  Dividends here are
// element and item indices checked on the host to stay below 2^31.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d) {   // host side, d >= 1
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return {d, uint32_t(m), l};
}

__host__ __device__ inline uint32_t fdiv(uint32_t n, FastDiv f) {
    return (uint32_t((uint64_t(n) * f.m) >> 32) + n) >> f.l;
}

// Pack VEC elements into one 16-byte vector (used where a vector is gathered
// element by element).
template <typename T>
struct Pack16 {
    union {
        u32x4 v;
        T e[Vec<T>::n];
    };
};

template <typename T>
__device__ __forceinline__ float to_f32(T v) { return static_cast<float>(v); }

// fp32 -> storage type, round to nearest even (the hardware default mode).
template <typename T>
__device__ __forceinline__ T from_f32(float v) { return static_cast<T>(v); }

// 16-bit NHWC small-window kernel: chunk geometry shared by the kernel, its
// filter pack and the planner.  `lead` zero-weight elements (0 or 1) come
// before each filter row's run of S*C elements, so that the run starts at an
// even element; cpr 8-element chunks cover lead + S*C.
struct Tile16Geom {
    int lead, cpr;
};
__host__ __device__ inline Tile16Geom tile16_geom(int C, int S, int pw) {
    const int lead = (pw * C) & 1;
    return {lead, (lead + S * C + 7) / 8};
}

// Workgroups of that kernel resident per CU (its persistent grid is this many
// per CU): 4*tn channels per lane and the filter in registers leave room
// for two waves per SIMD at tn = 4, three at tn = 2.
__host__ __device__ constexpr int tile16_wgs_per_cu(int tn) { return tn == 4 ? 2 : 3; }

// A row i of the 16 x 32 filter fragment of channel block jb holds output
// channel (i/4)*4*TN + jb*4 + i%4, so that the accumulator lane group g
// (rows 4g .. 4g+3 of every block) ends up with channels g*4*TN .. g*4*TN +
// 4*TN - 1 of its pixel.
__host__ __device__ inline int tile16_channel(int i, int jb, int tn) { return (i / 4) * 4 * tn + jb * 4 + (i % 4); }

}  // namespace convlower
