/*
 * convlower.h -- forward 2-D convolution lowered to a dense contraction on
 * AMD Instinct MI355X (gfx950): im2win window strips or explicit im2col
 * columns, then an LDS-staged MFMA contraction with a fused bias epilogue.
 *
 * The operation (cross-correlation, zero padding):
 *
 *   y[n,k,p,q] = b[k] + sum_{c<C, r<R, s<S}
 *                x[n, c, p*sh - ph + r*dh, q*sw - pw + s*dw] * w[k, c, r, s]
 *   P = floor((H + 2 ph - dh (R-1) - 1) / sh) + 1,  Q likewise,
 *
 * as described in "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a
 * Custom PyTorch Extension" (section "Transforming Conv2D into im2col and
 * GEMM": the output matrix is the reshaped filter matrix times the im2col
 * matrix of overlapping input windows), with the window-strip layout of
 * "Enabling Memory-efficient Im2win Convolution with Multi-precision Support
 * on GPU CUDA and Tensor Cores" (abstract: contiguous memory access for every
 * kernel size, lower memory than explicit im2col).
 *
 * Conventions shared by every entry point
 *  - All tensors are dense and packed (no strides).  layout CONV_NCHW means
 *    x is NCHW, w is KCRS and y is NKPQ; CONV_NHWC means x NHWC, w KRSC,
 *    y NPQK.  x, w, bias and y share one storage type; products are formed
 *    from the stored values and accumulated in fp32; y is rounded to the
 *    storage type once, round-to-nearest-even, after the bias is added.
 *  - x, w, bias, y and ws are DEVICE pointers owned by the caller.  x, w, y
 *    and ws must be 16-byte aligned; bias must be aligned to its element.
 *    y must not overlap x, w, bias or ws.
 *  - The library never allocates device memory, never copies between host
 *    and device and never synchronises -- with one exception, conv_tune,
 *    which times candidate plans and therefore waits for its own timing
 *    events.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *    default stream) and runs asynchronously; errors found on the host are
 *    returned before anything is enqueued, launch failures come back as
 *    CONV_ERR_HIP, and faults inside a kernel surface at the caller's next
 *    synchronisation.
 *  - There is no fallback: a case the kernels do not cover returns
 *    CONV_ERR_UNSUPPORTED and nothing runs.
 *  - A descriptor is immutable after creation (conv_tune returns a new one);
 *    one descriptor may be used from several threads and streams at once if
 *    each call has its own ws.
 *  - No entry point reads the process environment: a plan other than the
 *    default is only ever asked for explicitly (conv_create_desc_forced).
 */
#ifndef CONVLOWER_H
#define CONVLOWER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CONV_OK = 0,
    CONV_ERR_INVALID_ARG = -1,     /* sizes, strides, enum values out of range */
    CONV_ERR_UNSUPPORTED = -2,     /* valid convolution the kernels do not cover */
    CONV_ERR_NULL_PTR = -3,        /* a required pointer is NULL */
    CONV_ERR_NOT_DEVICE_PTR = -4,  /* a tensor pointer is not device memory */
    CONV_ERR_MISALIGNED = -5,      /* a tensor pointer breaks the alignment rule */
    CONV_ERR_HIP = -6,             /* the HIP runtime reported an error */
    CONV_ERR_OOM = -7              /* host allocation of a descriptor failed */
} conv_status_t;

typedef enum { CONV_NCHW = 0, CONV_NHWC = 1 } conv_layout_t;
typedef enum { CONV_F32 = 0, CONV_F16 = 1, CONV_BF16 = 2 } conv_dtype_t;

/* How the input is lowered before the contraction.
 *  CONV_ALGO_IM2WIN  for each (image n, output row p) one contiguous window
 *                    strip Win[n][p][j][r*C + c] over the W_used padded input
 *                    columns j the row's windows touch; a GEMM row (n,p,q) is
 *                    then the run of S strip columns starting at q*sw
 *                    (every dw-th column), so overlapping windows share
 *                    storage (the im2win layout).
 *  CONV_ALGO_IM2COL  explicit im2col: one materialised row per output pixel,
 *                    Col[(n,p,q)][s][r*C + c] (the baseline the im2win
 *                    workspace is compared against).
 *  CONV_ALGO_IMPLICIT the contraction gathers each output pixel's window
 *                    straight from x into its LDS tile (zero outside the
 *                    image), in the filter's own order -- (c, r, s) for KCRS,
 *                    (r, s, c) for KRSC -- so neither a lowered buffer nor a
 *                    packed filter is written: the workspace is 0 bytes and a
 *                    call is one kernel launch.
 * For 1x1 kernels on NHWC input with no padding, IM2WIN and IM2COL read x in
 * place and use no lowering workspace. */
typedef enum { CONV_ALGO_IM2WIN = 0, CONV_ALGO_IM2COL = 1, CONV_ALGO_IMPLICIT = 2 } conv_algo_t;

typedef struct {
    int64_t N, C, H, W;        /* input: batch, channels, height, width */
    int64_t K, R, S;           /* filter: output channels, kernel height, kernel width */
    int32_t stride_h, stride_w;
    int32_t pad_h, pad_w;      /* symmetric zero padding per dimension */
    int32_t dil_h, dil_w;
    conv_layout_t layout;
    conv_dtype_t dtype;
    conv_algo_t algo;
} conv_params_t;

typedef struct conv_desc* conv_desc_t;   /* opaque; owned by the library */

/* What a descriptor decided: extents, GEMM shape, workspace layout, tiling.
 * Filled by conv_plan_info; for reporting and for tests of the layouts. */
typedef struct {
    int64_t P, Q;              /* output extents */
    int64_t M;                 /* GEMM rows = N*P*Q */
    int64_t Kg;                /* contraction length of the definition = C*R*S */
    int64_t W_used;            /* padded input columns one output row's windows touch */
    int64_t RCp;               /* lowered window row: R*C rounded up to a 16-byte multiple of
                                * elements; R*C itself for fp32 when that is not a whole
                                * number of vectors (unpadded rows, read element by element) */
    int64_t Kl;                /* lowered contraction length = S*RCp (zeros in the padding) */
    uint64_t ws_bytes;         /* total workspace the caller must pass */
    uint64_t ws_filter_offset, ws_filter_bytes;    /* packed filter Bp[K][Kl] */
    uint64_t ws_lowered_offset, ws_lowered_bytes;  /* window strips or im2col rows */
    uint64_t im2win_bytes;     /* N*P*W_used*RCp*elem: im2win strip bytes for this shape */
    uint64_t im2col_bytes;     /* N*P*Q*C*R*S*elem: the plain explicit im2col matrix */
    int32_t lowering_elided;   /* 1: x is read in place (1x1 NHWC, no padding) */
    int32_t tile_m, tile_n, tile_k;  /* contraction tile chosen for this shape */
    int32_t elem_bytes;
    /* contraction kernel: 0 register-staged tiles, 1 LDS-DMA pipeline (two
     * waves per SIMD), 2 LDS-DMA pipeline with one wave per SIMD and 32x32
     * MFMA tiles, 3 fp32 NCHW windows, 4 input row strips staged in LDS,
     * 5 the same strips with the filter streamed into registers from a copy
     * in MFMA fragment order (that copy is the workspace's filter part),
     * 6 fp32 NCHW row strips loaded 16 bytes per lane, filter streamed the
     * same way, 7 fp32 NCHW small windows (C*R*S <= 64, K <= 64): input rows
     * staged once per block of output rows, whole filter in registers,
     * 8 16-bit NHWC small windows (the stem layers: C*sw and W*C even, unit
     * horizontal dilation, K <= 64): the same staging, each filter row's
     * window part read as one contiguous run, filter in registers from a
     * copy in MFMA fragment order, 9 the LDS-DMA pipeline of 1 in stream-K
     * form: a persistent grid whose workgroups take equal ranges of the
     * (tile, contraction step) pairs, a tile split between workgroups summed
     * in contraction order from fp32 slots in the workspace's partial area
     * (one tile_m*tile_n slot and one flag per workgroup), taken only when
     * named (conv_create_desc_forced) or kept by conv_tune, 10 the strips of
     * 5 with the taps of a filter row unrolled at compile time (filter widths
     * 3, 5, 7, 9, 11; unit horizontal dilation), strip rows padded to 80
     * bytes and pixels dealt to lanes so that fragment reads are
     * conflict-free at fixed offsets, 11 fp32 NCHW per-tap planes: for a
     * filter row and 16 input channels, each (channel, tap) element of the
     * tile's pixels gathered by 4-byte LDS-DMA loads into a plane of its own
     * (any padding, stride and dilation; filter widths 2 and 3; C % 16 == 0),
     * read without bank conflicts, filter streamed as for 6, 12 the
     * unrolled-tap strips of 10 on 16x16x32 MFMAs (the same 80-byte strip
     * rows; the filter copy in 16x16x32 fragment order), 13 the strips of 12
     * with each tap's filter fragments loaded once per workgroup into a ring
     * of LDS slots a few taps ahead and read from there by every wave,
     * 14 16-bit NHWC 1x1 layers with unit stride, no padding, C of 32, 64
     * or 128 and K <= 128: a persistent grid whose waves stream 16-pixel
     * blocks of x (several in flight each) against the filter held in LDS;
     * kernel_variant indexes that kernel's compiled tile shapes (for 9 the
     * shapes of 1) */
    int32_t kernel, kernel_variant;
    /* split contraction (kernels 1 and 2): ksplit workgroups share each output
     * tile, each over a contiguous range of the contraction, their fp32
     * partial sums [ksplit][N*P*Q*K] in the output layout at
     * ws_partial_offset; 1 = no split (ws_partial_bytes 0) */
    uint64_t ws_partial_offset, ws_partial_bytes;
    int32_t ksplit;
    /* order in which the workgroups of kernel 1 take the (split, output tile)
     * pairs (conv_tile_order_t); 0 for the other kernels */
    int32_t tile_order;
} conv_plan_info_t;

/* Tile orders of the pipelined kernel (conv_plan_info_t.tile_order, the
 * fourth field of a forced plan).  The GPU deals workgroups to its eight XCDs,
 * each with its own L2, round robin; LINEAR leaves consecutive tiles on
 * different XCDs, the other orders give each XCD one contiguous range of the
 * (split, tile row, tile column) sequence: row-major, row-major with odd tile
 * rows right to left (serpentine: consecutive tiles always share an operand
 * panel), or column-major.  "Enabling Memory-efficient Im2win Convolution
 * ...", abstract (the order of memory accesses as a tuning dimension);
 * "GPU-Accelerating MSCRED ...", section "Future Work" (further tile and
 * thread-block configurations). */
typedef enum {
    CONV_TILE_LINEAR = 0,
    CONV_TILE_XCD_ROWS = 1,
    CONV_TILE_XCD_SERPENT = 2,
    CONV_TILE_XCD_COLS = 3
} conv_tile_order_t;

/* Validate *p and build a descriptor.  "GPU-Accelerating MSCRED ...",
 * section "Integrating the CUDA Implementation with PyTorch" (the extension
 * checks tensor dimensions, data types, device placement and contiguity, and
 * handles errors) and section "Transforming Conv2D into im2col and GEMM" (the
 * sizes of the lowered matrix and of the output feature map follow from the
 * convolution's parameters): all of that is decided here, once, on the host.
 * Host only: no HIP call is made, so it works without a GPU.  Errors:
 * CONV_ERR_NULL_PTR (p or out NULL), CONV_ERR_INVALID_ARG (N < 0,
 * C/H/W/K/R/S <= 0, stride or dilation <= 0, padding < 0, bad enum, or a
 * kernel that does not fit the padded input, i.e. P or Q <= 0),
 * CONV_ERR_UNSUPPORTED (sizes beyond the 32-bit index ranges the kernels
 * use), CONV_ERR_OOM.  On success *out owns a descriptor the caller must
 * release with conv_destroy_desc. */
conv_status_t conv_create_desc(const conv_params_t* p, conv_desc_t* out);

/* As conv_create_desc, with the contraction kernel named explicitly: plan is
 * "<kernel>:<variant>", "<kernel>:<variant>:<ksplit>" or
 * "<kernel>:<variant>:<ksplit>:<tile order>" with kernel one of reg, dma,
 * wide, nchw, strip, striprb, nchwstrip, nchwtile, tile16, streamk,
 * striprb2, nchwtaps, striprb3, striprb4, stream1x1 (the numbering of conv_plan_info_t.kernel,
 * in that order) and
 * variant an index
 * into that kernel's compiled tile shapes; ksplit (1-8) splits the
 * contraction of the dma and wide kernels; tile order (conv_tile_order_t)
 * applies to the dma kernel.  "GPU-Accelerating MSCRED ...",
 * section "Engineering Challenges" (kernel configuration: thread-block
 * dimensions and tile sizes change occupancy, memory access and work
 * distribution, so they are measured, not assumed).  For tests and tuning: a
 * plan that does not take this convolution, or a malformed string, leaves
 * the default plan (conv_plan_info says which was kept).  plan == NULL is
 * conv_create_desc.  Host only; errors as conv_create_desc. */
conv_status_t conv_create_desc_forced(const conv_params_t* p, const char* plan, conv_desc_t* out);

/* Release a descriptor (NULL is accepted and ignored; a pointer that is not a
 * live descriptor returns CONV_ERR_INVALID_ARG).  "GPU-Accelerating MSCRED
 * ...", section "Engineering Challenges" (memory management: what is
 * allocated is released).  Host only. */
conv_status_t conv_destroy_desc(conv_desc_t d);

/* Bytes of device workspace conv2d_fwd needs for this descriptor (may be 0).
 * "GPU-Accelerating MSCRED ...", section "Engineering Challenges" (the
 * im2col transformation creates intermediate data whose allocation, reuse and
 * release must be managed): the caller allocates this many bytes, may reuse
 * them for any call with a descriptor that needs no more, and frees them;
 * the library never allocates.  The figure is what the plan lowers (im2win
 * strips: "Enabling Memory-efficient Im2win Convolution ...", abstract; or
 * explicit im2col rows) plus any packed filter or split-contraction partial
 * sums.  Host only. */
conv_status_t conv_workspace_size(conv_desc_t d, size_t* bytes);

/* Output extents P, Q (floor formula above; "GPU-Accelerating MSCRED ...",
 * section "Transforming Conv2D into im2col and GEMM": the product is
 * reshaped into the output feature map).  Host only. */
conv_status_t conv_output_dims(conv_desc_t d, int64_t* P, int64_t* Q);

/* The descriptor's plan (see conv_plan_info_t): "GPU-Accelerating MSCRED
 * ...", section "Engineering Challenges" (measuring the correct bottleneck:
 * the choice a measurement is about must be visible).  Host only. */
conv_status_t conv_plan_info(conv_desc_t d, conv_plan_info_t* info);

/* The whole forward convolution: conv_pack_filter, conv_lower_input and
 * conv_contract enqueued in that order on `stream`.  "GPU-Accelerating MSCRED
 * ...", section "Transforming Conv2D into im2col and GEMM" (overlapping input
 * windows become the columns of a matrix that the reshaped filter matrix
 * multiplies; the result is reshaped into the output feature map) and
 * section "Global Memory and Shared Memory" (reusable tiles staged in on-chip
 * memory); "Enabling Memory-efficient Im2win Convolution ...", abstract (the
 * window layout, asynchronous data movement, fp32 and half-precision
 * arithmetic).  Errors (all found before anything is enqueued):
 * CONV_ERR_INVALID_ARG (not a live descriptor, or a ConvLSTM one),
 * CONV_ERR_NULL_PTR, CONV_ERR_NOT_DEVICE_PTR, CONV_ERR_MISALIGNED; a launch
 * failure returns CONV_ERR_HIP.
 *   x     input, N*C*H*W elements in the descriptor's layout
 *   w     filter, K*C*R*S elements (KCRS or KRSC)
 *   bias  K elements, or NULL for no bias
 *   y     output, N*K*P*Q elements (NKPQ or NPQK); fully overwritten
 *   ws    at least conv_workspace_size bytes (NULL iff that size is 0); its
 *         contents on entry are ignored and on return are unspecified
 * N == 0 is accepted and enqueues nothing. */
conv_status_t conv2d_fwd(conv_desc_t d, const void* x, const void* w, const void* bias, void* y,
                         void* ws, void* stream);

/* Workspace limit of conv2d_fwd_noalloc, in bytes (64 MiB). */
#define CONV_NOALLOC_SCRATCH_BYTES (64ull << 20)

/* conv2d_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * caller still passes x, w, bias and y (as for conv2d_fwd); the workspace is
 * instead a fixed array of CONV_NOALLOC_SCRATCH_BYTES in device memory that
 * the library holds on each GPU it runs on until the process ends (its address
 * is looked up on the first call on a device).  No hipMalloc, hipFree or
 * other allocating call is made.  Every call on one GPU shares that GPU's
 * array: calls that overlap in time on one GPU (other streams, other
 * threads) race on it and must not be issued; calls in sequence on one stream
 * are safe (each kernel writes every scratch byte it reads before reading
 * it, so nothing is cleared between calls).  Errors as conv2d_fwd, and
 * CONV_ERR_UNSUPPORTED (nothing enqueued) when conv_workspace_size(d) exceeds
 * CONV_NOALLOC_SCRATCH_BYTES (for scale: the fused path of a 3x3, 512- to
 * 512-channel layer over 64 images of 7x7 keeps 12.8 MB of split-contraction
 * partial sums; lowered im2win / im2col buffers of large layers exceed it). */
conv_status_t conv2d_fwd_noalloc(conv_desc_t d, const void* x, const void* w, const void* bias, void* y,
                                 void* stream);

/* Stage 1 of conv2d_fwd: reorder w into the packed contraction operand
 * Bp[k][s*RCp + r*C + c] in ws (zeros in the RCp padding) -- the "reshaped
 * filter matrix" of "GPU-Accelerating MSCRED ...", section "Transforming
 * Conv2D into im2col and GEMM" -- or, for the register-streamed and
 * small-window kernels, into the order their MFMAs consume it.  A no-op when
 * the plan reads w in place (the fused path's pipelined and streaming 1x1
 * kernels, the variants of kernel 13 that read the KRSC rows, and NHWC with
 * R == 1 or S == 1 and C a multiple of the 16-byte vector).  Pointer rules
 * and errors as conv2d_fwd. */
conv_status_t conv_pack_filter(conv_desc_t d, const void* w, void* ws, void* stream);

/* Stage 2: lower x into ws -- im2win strips ("Enabling Memory-efficient
 * Im2win Convolution ...", abstract) or im2col rows ("GPU-Accelerating MSCRED
 * ...", section "Transforming Conv2D into im2col and GEMM": overlapping
 * windows copied into an intermediate matrix), per the descriptor's
 * algorithm.  A no-op when the lowering is elided and for
 * CONV_ALGO_IMPLICIT.  Pointer rules and errors as conv2d_fwd. */
conv_status_t conv_lower_input(conv_desc_t d, const void* x, void* ws, void* stream);

/* Stage 3: the MFMA contraction over the lowered operand and packed filter
 * with the fused epilogue y = round(acc + bias[k]) ("GPU-Accelerating MSCRED
 * ...", sections "Transforming Conv2D into im2col and GEMM" -- the matrix
 * product and the reshape into the output map -- and "Global Memory and
 * Shared Memory" -- tiles reused from on-chip memory).  Reads ws written by
 * stages 1 and 2; reads x in place when the lowering is elided and w in place
 * when the pack is a no-op.  When the plan splits the contraction
 * (conv_plan_info_t.ksplit > 1) it also writes the fp32 partial sums into
 * ws's partial area and then enqueues their reduction (sum in split order,
 * plus bias, rounded once). */
conv_status_t conv_contract(conv_desc_t d, const void* x, const void* w, const void* bias, void* y,
                            void* ws, void* stream);

/* ---------------------------------------------------------------- ConvLSTM step
 * "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
 * Extension", sections "MSCRED and ConvLSTM Architecture" and "Why the
 * Encoder Improved More Than ConvLSTM": after the encoder, ConvLSTM layers
 * carry the encoded maps through time and become the bottleneck.  The pages
 * give no cell equations; this library reads the cell as the standard one
 * without peepholes, its four gates from one convolution over the channel
 * concatenation of the step's input and the previous hidden state:
 *   z   = conv(concat(x, h_prev), w) + bias     (4*Kh channels, order i, f, g, o)
 *   c_t = sigmoid(z_f) * c_prev + sigmoid(z_i) * tanh(z_g)
 *   h_t = sigmoid(z_o) * tanh(c_t)
 * The gate convolution runs through this library's lowering (im2win or
 * im2col, reading x and h_prev in place of their concatenation) and MFMA
 * contraction; the cell update is fused into the contraction's epilogue. */

/* Plan a ConvLSTM step.  p describes the gate convolution: C = c_x + Kh
 * input channels (c_x from x, Kh from h_prev), K = 4*Kh, stride 1, and
 * padding / dilation that keep the output H x W; layout CONV_NCHW, dtype
 * CONV_F32, algo CONV_ALGO_IM2WIN or CONV_ALGO_IM2COL.  Kh must be a multiple
 * of 16.  Host only; CONV_ERR_INVALID_ARG for inconsistent sizes,
 * CONV_ERR_UNSUPPORTED for another layout, dtype or algorithm.  The
 * descriptor is used with conv_lstm_step (the plain-convolution entry points
 * reject it) and conv_workspace_size / conv_output_dims / conv_plan_info /
 * conv_destroy_desc. */
conv_status_t conv_lstm_create_desc(const conv_params_t* p, int64_t c_x, conv_desc_t* out);

/* One ConvLSTM step on `stream`; device pointers, caller-owned, NCHW fp32,
 * 16-byte aligned (bias 4-byte):
 *   x       N*c_x*H*W             h_prev, c_prev   N*Kh*H*W
 *   w       4*Kh*(c_x+Kh)*R*S (KCRS, gate blocks in the order i, f, g, o)
 *   bias    4*Kh, or NULL
 *   h_out, c_out   N*Kh*H*W, fully overwritten; must not alias the inputs
 *   ws      at least conv_workspace_size bytes
 * N == 0 enqueues nothing. */
conv_status_t conv_lstm_step(conv_desc_t d, const void* x, const void* h_prev, const void* c_prev, const void* w,
                             const void* bias, void* h_out, void* c_out, void* ws, void* stream);

/* ---------------------------------------------------------------- tile choice
 * The pages sweep tile sizes and thread-block shapes ("GPU-Accelerating
 * MSCRED ...", section "CUDA Kernel Design"; the im2win abstract) without
 * fixing a rule.  conv_tune times, on the caller's tensors, the descriptor's
 * current plan and every other compiled contraction kernel and tile variant
 * that takes its convolution and whose workspace fits ws_bytes (the pipelined
 * and wide-tile kernels' variants each without a split contraction and with 2
 * and 4 splits), then, when the fastest is the pipelined kernel, that plan in
 * each tile order, and keeps the fastest. */
typedef struct {
    int32_t candidates;       /* plans timed, the current one included */
    int32_t kernel;           /* the plan kept (conv_plan_info_t numbering) */
    int32_t kernel_variant;
    float default_ms;         /* ms per conv2d_fwd-equivalent call, the plan d had on entry */
    float best_ms;            /* ms per call of the plan kept */
    int32_t ksplit;           /* its split contraction (conv_plan_info_t.ksplit) */
    int32_t tile_order;       /* its tile order (conv_plan_info_t.tile_order) */
} conv_tune_result_t;

/* Tune the plan of d (not a ConvLSTM descriptor) with reps timed calls per
 * candidate, on `stream`, with the same pointer rules as conv2d_fwd; ws_bytes
 * is the size of ws (at least conv_workspace_size(d)); only candidates whose
 * workspace fits ws_bytes are timed.  The one entry point that synchronises:
 * it blocks the calling thread until its timing events are in.  d itself is
 * not changed (other users of it are unaffected); the plan kept is returned
 * in *tuned, a new descriptor the caller releases with conv_destroy_desc --
 * query its conv_workspace_size, which is never above ws_bytes.  On return y
 * holds the output of the last candidate run and *result says what was kept.
 * Errors as conv2d_fwd, CONV_ERR_NULL_PTR for a NULL tuned or result,
 * CONV_ERR_INVALID_ARG for reps < 1 or ws_bytes below the current workspace
 * size, CONV_ERR_OOM; on an error *tuned is NULL. */
conv_status_t conv_tune(conv_desc_t d, const void* x, const void* w, const void* bias, void* y, void* ws,
                        size_t ws_bytes, int32_t reps, void* stream, conv_desc_t* tuned,
                        conv_tune_result_t* result);

/* Static English text for a status code ("GPU-Accelerating MSCRED ...",
 * section "Integrating the CUDA Implementation with PyTorch": error handling
 * at the boundary).  Never NULL; "unknown status" for other values. */
const char* conv_status_string(conv_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* CONVLOWER_H */
