// Peak microbenchmarks (declarations and argument rules in include/convpeak.h):
// the MFMA rate of each instruction the contraction kernels use, from a loop
// of independent MFMAs on register operands (no memory traffic at all), the
// shader clock sustained meanwhile, and the bandwidth of a streaming copy.
// What the convolution kernels reach is then stated against what this GPU
// sustains as well as against the published figures.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/convpeak.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Independent accumulators per iteration: enough that no MFMA waits for the
// result of the one before it on the same accumulator.
constexpr int kAcc32 = 4;    // 32x32 tiles: 4 x 16 VGPRs
constexpr int kAcc16 = 8;    // 16x16 tiles: 8 x 4 VGPRs

template <int KIND>
struct PeakOp;

template <>
struct PeakOp<PEAK_MFMA_F32_16X16X4> {
    static constexpr int NACC = kAcc16;
    static constexpr int64_t FLOPS = 2 * 16 * 16 * 4;
    using Acc = f32x4;
    using Op = float;
    static __device__ Op operand(uint32_t seed) { return float(seed & 7) * 0.125f; }
    static __device__ Acc mma(Op a, Op b, Acc c) { return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0); }
};

template <int KIND>
struct Peak16 {
    static __device__ u32x4 operand(uint32_t seed) {
        // small positive values in either 16-bit format: no overflow over the loop
        const uint32_t h = KIND == PEAK_MFMA_F16_32X32X16 || KIND == PEAK_MFMA_F16_16X16X32 ? 0x2000u : 0x3000u;
        const uint32_t v = (h | (seed & 0xff)) * 0x10001u;
        return u32x4{v, v ^ 0x10001u, v, v ^ 0x20002u};
    }
};

template <>
struct PeakOp<PEAK_MFMA_F16_32X32X16> : Peak16<PEAK_MFMA_F16_32X32X16> {
    static constexpr int NACC = kAcc32;
    static constexpr int64_t FLOPS = 2 * 32 * 32 * 16;
    using Acc = f32x16;
    using Op = u32x4;
    static __device__ Acc mma(Op a, Op b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

template <>
struct PeakOp<PEAK_MFMA_BF16_32X32X16> : Peak16<PEAK_MFMA_BF16_32X32X16> {
    static constexpr int NACC = kAcc32;
    static constexpr int64_t FLOPS = 2 * 32 * 32 * 16;
    using Acc = f32x16;
    using Op = u32x4;
    static __device__ Acc mma(Op a, Op b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};

template <>
struct PeakOp<PEAK_MFMA_F16_16X16X32> : Peak16<PEAK_MFMA_F16_16X16X32> {
    static constexpr int NACC = kAcc16;
    static constexpr int64_t FLOPS = 2 * 16 * 16 * 32;
    using Acc = f32x4;
    using Op = u32x4;
    static __device__ Acc mma(Op a, Op b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
};

template <>
struct PeakOp<PEAK_MFMA_BF16_16X16X32> : Peak16<PEAK_MFMA_BF16_16X16X32> {
    static constexpr int NACC = kAcc16;
    static constexpr int64_t FLOPS = 2 * 16 * 16 * 32;
    using Acc = f32x4;
    using Op = u32x4;
    static __device__ Acc mma(Op a, Op b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
};

// At least two workgroups per CU: with the bare 256-thread bound the
// compiler allocates the 16x16 accumulators to AGPRs and copies them through
// VGPRs on every iteration, which chains the MFMAs; with this bound the loop
// is the MFMAs alone (checked in the ISA).
template <int KIND>
__global__ void __launch_bounds__(256, 2) peak_mfma_kernel(int64_t iters, uint64_t* clocks) {
    using P = PeakOp<KIND>;
    const uint32_t lane = threadIdx.x & 63;
    const bool first = threadIdx.x == 0;
    uint64_t c0 = 0, r0 = 0;
    if (first) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const typename P::Op a = P::operand(lane), b = P::operand(lane * 7 + blockIdx.x);
    typename P::Acc acc[P::NACC];
#pragma unroll
    for (int i = 0; i < P::NACC; ++i) acc[i] = typename P::Acc{};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < P::NACC; ++i) acc[i] = P::mma(a, b, acc[i]);
    }
    // every element of every accumulator feeds the checksum
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < P::NACC; ++i)
#pragma unroll
        for (int e = 0; e < int(sizeof(typename P::Acc) / sizeof(float)); ++e) sum += acc[i][e];
    if (first) {
        const uint64_t c1 = __builtin_amdgcn_s_memtime();
        const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
        uint64_t* o = clocks + int64_t(blockIdx.x) * 8;
        o[0] = c0;
        o[1] = c1;
        o[2] = r0;
        o[3] = r1;
        o[4] = __float_as_uint(sum);
    }
}

// Each workgroup moves spans of 256 * U contiguous vectors (lane i takes
// vectors i, i + 256, ... of the span, so every load instruction of the
// workgroup covers 4 KiB of consecutive bytes); spans are dealt out
// grid-stride.
__global__ void __launch_bounds__(256) peak_copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t nvec) {
    constexpr int U = 4;   // vectors in flight per lane
    constexpr int64_t SPAN = 256 * U;
    for (int64_t base = int64_t(blockIdx.x) * SPAN; base < nvec; base += int64_t(gridDim.x) * SPAN) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            v[u] = i < nvec ? __builtin_nontemporal_load(src + i) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + threadIdx.x;
            if (i < nvec) __builtin_nontemporal_store(v[u], dst + i);
        }
    }
}

}  // namespace

extern "C" {

int64_t convpeak_mfma_flops_per_iter(int32_t kind) {
    switch (kind) {
        case PEAK_MFMA_F32_16X16X4: return PeakOp<PEAK_MFMA_F32_16X16X4>::FLOPS * PeakOp<PEAK_MFMA_F32_16X16X4>::NACC;
        case PEAK_MFMA_F16_32X32X16: return PeakOp<PEAK_MFMA_F16_32X32X16>::FLOPS * PeakOp<PEAK_MFMA_F16_32X32X16>::NACC;
        case PEAK_MFMA_BF16_32X32X16:
            return PeakOp<PEAK_MFMA_BF16_32X32X16>::FLOPS * PeakOp<PEAK_MFMA_BF16_32X32X16>::NACC;
        case PEAK_MFMA_F16_16X16X32: return PeakOp<PEAK_MFMA_F16_16X16X32>::FLOPS * PeakOp<PEAK_MFMA_F16_16X16X32>::NACC;
        case PEAK_MFMA_BF16_16X16X32:
            return PeakOp<PEAK_MFMA_BF16_16X16X32>::FLOPS * PeakOp<PEAK_MFMA_BF16_16X16X32>::NACC;
        default: return 0;
    }
}

int convpeak_mfma(int32_t kind, int64_t iters, int32_t blocks, void* clocks, void* stream) {
    if (iters < 1 || blocks < 1 || blocks > 65535 || !clocks) return -1;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    uint64_t* c = static_cast<uint64_t*>(clocks);
    switch (kind) {
        case PEAK_MFMA_F32_16X16X4: peak_mfma_kernel<PEAK_MFMA_F32_16X16X4><<<blocks, 256, 0, st>>>(iters, c); break;
        case PEAK_MFMA_F16_32X32X16: peak_mfma_kernel<PEAK_MFMA_F16_32X32X16><<<blocks, 256, 0, st>>>(iters, c); break;
        case PEAK_MFMA_BF16_32X32X16:
            peak_mfma_kernel<PEAK_MFMA_BF16_32X32X16><<<blocks, 256, 0, st>>>(iters, c);
            break;
        case PEAK_MFMA_F16_16X16X32: peak_mfma_kernel<PEAK_MFMA_F16_16X16X32><<<blocks, 256, 0, st>>>(iters, c); break;
        case PEAK_MFMA_BF16_16X16X32:
            peak_mfma_kernel<PEAK_MFMA_BF16_16X16X32><<<blocks, 256, 0, st>>>(iters, c);
            break;
        default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int convpeak_wall_clock_khz(int64_t* khz) {
    if (!khz) return -1;
    int dev = 0, rate = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -6;
    if (hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return -6;
    *khz = rate;
    return 0;
}

int convpeak_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16 || reinterpret_cast<uintptr_t>(dst) % 16)
        return -1;
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return -1;
    const int64_t nvec = int64_t(bytes / 16);
    if (nvec == 0) return 0;
    const int64_t want = (nvec + 1023) / 1024;
    const int blocks = int(want < 256 * 8 ? want : 256 * 8);   // 8 workgroups per CU
    peak_copy_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const u32x4*>(src),
                                                                          static_cast<u32x4*>(dst), nvec);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
