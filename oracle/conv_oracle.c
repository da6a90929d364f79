/*
 * conv_oracle.c -- reference forward 2-D convolution in double precision.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: it exists so that the GPU library can be checked against a
 * plain, slow and obviously correct computation.  Only the test suite, the
 * package smoke check and the CPU-baseline leg of the benchmark use it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * What it computes.  "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a
 * Custom PyTorch Extension", section "Where the Performance Bottleneck
 * Appeared", describes the CPU convolution as nested loops over batch
 * elements, output filters, spatial positions, input channels and kernel
 * dimensions; section "Transforming Conv2D into im2col and GEMM" says a
 * kernel is applied to overlapping regions of the input feature map.  The
 * plainest reading, and the one PyTorch (the reference those pages compare
 * against) uses, is the cross-correlation
 *
 *   y[n,k,p,q] = b[k] + sum_{c<C} sum_{r<R} sum_{s<S}
 *                x[n, c, p*sh - ph + r*dh, q*sw - pw + s*dw] * w[k, c, r, s]
 *
 * with x taken as zero outside [0,H) x [0,W), and output extents
 *   P = floor((H + 2 ph - dh (R-1) - 1) / sh) + 1,   Q likewise.
 *
 * It is computed here as seven loops (n, k, p, q, c, r, s) in that order,
 * with one fp64 accumulator per output.  Inputs stored as fp32, fp16 or bf16
 * are first decoded to double exactly (every value of those formats is a
 * double), so every product is exact and the only rounding is the fp64
 * summation.  Alongside y it can return yabs = |b[k]| + sum |x * w|, the
 * scale against which a computed result's error is judged.
 *
 * Threads split the (n, k) pairs; each output is still summed by one thread in
 * the fixed (c, r, s) order, so results do not depend on the thread count.
 *
 * Layouts: layout 0 = x NCHW, w KCRS, y NKPQ;  layout 1 = x NHWC, w KRSC,
 * y NPQK.  Storage types: 0 = fp32, 1 = fp16, 2 = bf16, 3 = fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
    int64_t N, C, H, W, K, R, S;
    int64_t stride_h, stride_w, pad_h, pad_w, dil_h, dil_w;
    int64_t layout;
    int64_t dtype;
} oracle_problem;

/* ---- exact decoding of the storage formats ---------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac + 1024), expo - 25);  /* 1.frac * 2^(expo-15) */
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
static double decode_bf16(uint16_t bits)
{
    int sign = bits >> 15;
    int expo = (bits >> 7) & 0xff;
    int frac = bits & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);                /* subnormal: frac * 2^-133 */
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac + 128), expo - 134);  /* 1.frac * 2^(expo-127) */
    return sign ? -v : v;
}

/* IEEE 754 binary32, read field by field rather than through a float cast. */
static double decode_f32(uint32_t bits)
{
    int sign = bits >> 31;
    int expo = (bits >> 23) & 0xff;
    int32_t frac = bits & 0x7fffff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -149);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(frac + 0x800000), expo - 150);
    return sign ? -v : v;
}

int oracle_decode(int64_t dtype, const void* src, int64_t count, double* dst)
{
    if (count < 0 || (count > 0 && (!src || !dst)))
        return -1;
    for (int64_t i = 0; i < count; ++i) {
        switch (dtype) {
        case 0: { uint32_t u; memcpy(&u, (const char*)src + 4 * i, 4); dst[i] = decode_f32(u); break; }
        case 1: { uint16_t u; memcpy(&u, (const char*)src + 2 * i, 2); dst[i] = decode_f16(u); break; }
        case 2: { uint16_t u; memcpy(&u, (const char*)src + 2 * i, 2); dst[i] = decode_bf16(u); break; }
        case 3: memcpy(&dst[i], (const char*)src + 8 * i, 8); break;
        default: return -1;
        }
    }
    return 0;
}

/* ---- problem checks and output extents --------------------------------- */

int oracle_output_dims(const oracle_problem* pr, int64_t* P, int64_t* Q)
{
    if (!pr || !P || !Q)
        return -1;
    if (pr->N < 0 || pr->C <= 0 || pr->H <= 0 || pr->W <= 0 || pr->K <= 0 || pr->R <= 0 || pr->S <= 0)
        return -1;
    if (pr->stride_h <= 0 || pr->stride_w <= 0 || pr->dil_h <= 0 || pr->dil_w <= 0 || pr->pad_h < 0 || pr->pad_w < 0)
        return -1;
    if (pr->layout != 0 && pr->layout != 1)
        return -1;
    int64_t span_h = pr->H + 2 * pr->pad_h - pr->dil_h * (pr->R - 1) - 1;
    int64_t span_w = pr->W + 2 * pr->pad_w - pr->dil_w * (pr->S - 1) - 1;
    if (span_h < 0 || span_w < 0)
        return -1;                          /* the kernel does not fit: no output */
    *P = span_h / pr->stride_h + 1;
    *Q = span_w / pr->stride_w + 1;
    return 0;
}

/* ---- element addressing, one function per tensor ----------------------- */

static int64_t x_index(const oracle_problem* pr, int64_t n, int64_t c, int64_t h, int64_t w)
{
    if (pr->layout == 0)
        return ((n * pr->C + c) * pr->H + h) * pr->W + w;
    return ((n * pr->H + h) * pr->W + w) * pr->C + c;
}

static int64_t w_index(const oracle_problem* pr, int64_t k, int64_t c, int64_t r, int64_t s)
{
    if (pr->layout == 0)
        return ((k * pr->C + c) * pr->R + r) * pr->S + s;
    return ((k * pr->R + r) * pr->S + s) * pr->C + c;
}

static int64_t y_index(const oracle_problem* pr, int64_t P, int64_t Q, int64_t n, int64_t k, int64_t p, int64_t q)
{
    if (pr->layout == 0)
        return ((n * pr->K + k) * P + p) * Q + q;
    return ((n * P + p) * Q + q) * pr->K + k;
}

/* ---- one output element: the three innermost loops --------------------- */

static double one_output(const oracle_problem* pr, const double* x, const double* w, const double* b,
                         int64_t n, int64_t k, int64_t p, int64_t q, double* abs_out)
{
    double acc = b ? b[k] : 0.0;
    double mag = b ? fabs(b[k]) : 0.0;
    for (int64_t c = 0; c < pr->C; ++c) {
        for (int64_t r = 0; r < pr->R; ++r) {
            int64_t h = p * pr->stride_h - pr->pad_h + r * pr->dil_h;
            for (int64_t s = 0; s < pr->S; ++s) {
                int64_t ww = q * pr->stride_w - pr->pad_w + s * pr->dil_w;
                int inside = h >= 0 && h < pr->H && ww >= 0 && ww < pr->W;
                double xv = inside ? x[x_index(pr, n, c, h, ww)] : 0.0;   /* zero padding */
                double prod = xv * w[w_index(pr, k, c, r, s)];
                acc += prod;
                mag += fabs(prod);
            }
        }
    }
    if (abs_out)
        *abs_out = mag;
    return acc;
}

/* ---- thread plumbing ---------------------------------------------------- */

typedef struct {
    const oracle_problem* pr;
    const double *x, *w, *b;
    int64_t P, Q;
    double *y, *yabs;
    const int64_t* pts;     /* NULL: full output; else npts rows of (n, k, p, q) */
    int64_t npts;
    int tid, nthreads;
} work_t;

static void* full_worker(void* arg)
{
    work_t* t = (work_t*)arg;
    const oracle_problem* pr = t->pr;
    int64_t slabs = pr->N * pr->K;
    for (int64_t slab = t->tid; slab < slabs; slab += t->nthreads) {
        int64_t n = slab / pr->K, k = slab % pr->K;
        for (int64_t p = 0; p < t->P; ++p) {
            for (int64_t q = 0; q < t->Q; ++q) {
                double mag;
                int64_t o = y_index(pr, t->P, t->Q, n, k, p, q);
                t->y[o] = one_output(pr, t->x, t->w, t->b, n, k, p, q, &mag);
                if (t->yabs)
                    t->yabs[o] = mag;
            }
        }
    }
    return NULL;
}

static void* point_worker(void* arg)
{
    work_t* t = (work_t*)arg;
    for (int64_t i = t->tid; i < t->npts; i += t->nthreads) {
        const int64_t* e = t->pts + 4 * i;
        double mag;
        t->y[i] = one_output(t->pr, t->x, t->w, t->b, e[0], e[1], e[2], e[3], &mag);
        if (t->yabs)
            t->yabs[i] = mag;
    }
    return NULL;
}

static int run_threads(work_t* proto, int nthreads, void* (*fn)(void*))
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    work_t jobs[256];
    int started = 0, rc = 0;
    for (int i = 0; i < nthreads; ++i) {
        jobs[i] = *proto;
        jobs[i].tid = i;
        jobs[i].nthreads = nthreads;
    }
    for (int i = 1; i < nthreads; ++i) {
        if (pthread_create(&th[i], NULL, fn, &jobs[i]) != 0) {
            rc = -2;
            break;
        }
        started = i;
    }
    if (rc != 0) {
        /* Run the slices whose threads did not start on this thread instead. */
        for (int i = started + 1; i < nthreads; ++i)
            fn(&jobs[i]);
        rc = 0;
    }
    fn(&jobs[0]);
    for (int i = 1; i <= started; ++i)
        pthread_join(th[i], NULL);
    return rc;
}

static int decode_operands(const oracle_problem* pr, const void* x, const void* w, const void* b,
                           double** xd, double** wd, double** bd)
{
    int64_t nx = pr->N * pr->C * pr->H * pr->W;
    int64_t nw = pr->K * pr->C * pr->R * pr->S;
    *xd = (double*)malloc(sizeof(double) * (size_t)(nx > 0 ? nx : 1));
    *wd = (double*)malloc(sizeof(double) * (size_t)nw);
    *bd = b ? (double*)malloc(sizeof(double) * (size_t)pr->K) : NULL;
    if (!*xd || !*wd || (b && !*bd))
        return -3;
    if (oracle_decode(pr->dtype, x, nx, *xd) || oracle_decode(pr->dtype, w, nw, *wd))
        return -1;
    if (b && oracle_decode(pr->dtype, b, pr->K, *bd))
        return -1;
    return 0;
}

int oracle_conv2d(const oracle_problem* pr, const void* x, const void* w, const void* b,
                  double* y, double* yabs, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pr, &P, &Q) != 0 || pr->dtype < 0 || pr->dtype > 3)
        return -1;
    if ((pr->N > 0 && (!x || !y)) || !w)
        return -1;
    double *xd = NULL, *wd = NULL, *bd = NULL;
    int rc = decode_operands(pr, x, w, b, &xd, &wd, &bd);
    if (rc == 0) {
        work_t proto = {pr, xd, wd, bd, P, Q, y, yabs, NULL, 0, 0, 1};
        rc = run_threads(&proto, nthreads, full_worker);
    }
    free(xd);
    free(wd);
    free(bd);
    return rc;
}

int oracle_conv2d_points(const oracle_problem* pr, const void* x, const void* w, const void* b,
                         const int64_t* nkpq, int64_t npts, double* y, double* yabs, int nthreads)
{
    int64_t P, Q;
    if (oracle_output_dims(pr, &P, &Q) != 0 || pr->dtype < 0 || pr->dtype > 3 || npts < 0)
        return -1;
    if (npts > 0 && (!x || !w || !nkpq || !y))
        return -1;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t* e = nkpq + 4 * i;
        if (e[0] < 0 || e[0] >= pr->N || e[1] < 0 || e[1] >= pr->K || e[2] < 0 || e[2] >= P || e[3] < 0 || e[3] >= Q)
            return -1;
    }
    double *xd = NULL, *wd = NULL, *bd = NULL;
    int rc = decode_operands(pr, x, w, b, &xd, &wd, &bd);
    if (rc == 0) {
        work_t proto = {pr, xd, wd, bd, P, Q, y, yabs, nkpq, npts, 0, 1};
        rc = run_threads(&proto, nthreads, point_worker);
    }
    free(xd);
    free(wd);
    free(bd);
    return rc;
}
