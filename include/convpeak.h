/*
 * convpeak.h -- measured peaks of the GPU the convolution library runs on:
 * the MFMA rate per storage type from a register-only loop, the shader clock
 * sustained under that load, and the HBM bandwidth of a plain streaming copy.
 *
 * "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
 * Extension", sections "Engineering Challenges" and "Engineering Lessons":
 * each optimisation is judged by profiling against what the hardware can
 * do.  The published MI355X figures are what the chip is specified for; these
 * kernels measure what this particular GPU sustains in the same run, so a
 * kernel's fraction of peak can be stated against both.
 *
 * Separate from libconvlower.so (built as libconvpeak.so): nothing on the
 * convolution path calls it.  Every pointer is a device pointer owned by the
 * caller; every call is asynchronous on `stream` (a hipStream_t, NULL = the
 * default stream) and makes no allocation and no synchronisation.  Return
 * values: 0 on success, -1 for an invalid argument, -6 when the HIP runtime
 * reports a launch error.
 */
#ifndef CONVPEAK_H
#define CONVPEAK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA instruction timed by convpeak_mfma. */
typedef enum {
    PEAK_MFMA_F32_16X16X4 = 0,    /* v_mfma_f32_16x16x4_f32:   2048 flop per instruction per wave */
    PEAK_MFMA_F16_32X32X16 = 1,   /* v_mfma_f32_32x32x16_f16:  32768 flop */
    PEAK_MFMA_BF16_32X32X16 = 2,  /* v_mfma_f32_32x32x16_bf16: 32768 flop */
    PEAK_MFMA_F16_16X16X32 = 3,   /* v_mfma_f32_16x16x32_f16:  16384 flop */
    PEAK_MFMA_BF16_16X16X32 = 4   /* v_mfma_f32_16x16x32_bf16: 16384 flop */
} peak_mfma_kind_t;

/* Flops one wave performs per loop iteration of convpeak_mfma for `kind`
 * (the instruction's flops times the independent accumulators per
 * iteration); 0 for an unknown kind.  Host only. */
int64_t convpeak_mfma_flops_per_iter(int32_t kind);

/* Launch `blocks` workgroups of 256 threads (4 waves), each wave running
 * `iters` iterations of independent MFMAs of `kind` on register operands.
 * Total flops = blocks * 4 * iters * convpeak_mfma_flops_per_iter(kind).
 * clocks: device buffer of blocks * 8 uint64 values; block b writes, from its
 * first wave, [b*8 + 0] = shader clock counter at the start, [+1] at the end,
 * [+2] = constant-rate wall clock at the start, [+3] at the end (see
 * convpeak_wall_clock_khz), [+4] = the bits of a sum of the accumulators (it
 * keeps the loop from being optimised away; its value means nothing).
 * iters >= 1, 1 <= blocks <= 65535. */
int convpeak_mfma(int32_t kind, int64_t iters, int32_t blocks, void* clocks, void* stream);

/* Frequency of the wall clock convpeak_mfma records, in kHz, for the current
 * device (hipDeviceAttributeWallClockRate).  Host only; -6 on a HIP error. */
int convpeak_wall_clock_khz(int64_t* khz);

/* dst[i] = src[i] for `bytes` bytes (a multiple of 16, both pointers 16-byte
 * aligned, no overlap): every lane moves 16-byte vectors, grid-stride. */
int convpeak_copy(const void* src, void* dst, size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CONVPEAK_H */
