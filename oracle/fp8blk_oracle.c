/*
 * fp8blk_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * FP8-blk dense linear (e4m3 codes with a 128x128 grid of e8m0 block scales,
 * multiplied against a short bf16 activation panel with f32 accumulation).
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this file's library. The
 * product path never does, and this file shares no source with it.
 *
 * Sources (docs.rs pages of the memra-engine crate):
 *   [Fp8Dense]  "Module dsv4_gpu" page, Structs, Fp8Dense: weights are e4m3
 *               codes [rows, cols] plus a 128x128 block-scale grid whose e8m0
 *               codes are powers of two, decoded to f32 on the host; code 0xFF
 *               is refused at load. The device twins form e4m3(code)*scale in
 *               registers, the same f32 the bf16 dequant slab holds, and keep
 *               the bf16 kernel's accumulation order, so both arms give
 *               identical bits.
 *   [Rungs]     "Module dsv4_gpu" page, module header (the rungs paragraph):
 *               quantized linears are dequantized to bf16 with a bit-level
 *               exactness refusal; bf16 enters only at the activation inputs;
 *               the products accumulate in f32.
 *   [dense_fp8] "Struct Dsv4Gpu" page, field dense_fp8: decode and verify read
 *               the FP8-blk linears as stored (e4m3 + f32 block scales).
 *   [batched]   "Struct Dsv4Gpu" page, spec_greedy_batched_with: each batched
 *               kernel gives the same bits as its single-position twin.
 *   [bf16_to_f32] "dflash.rs" source page, fn bf16_to_f32: a bf16 pattern is
 *               the high 16 bits of an f32.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - "e4m3" is the OCP FP8 E4M3 format (bias 7, max 448, subnormals, no
 *     infinities, NaN = S.1111.111); "e8m0" is 2^(c-127) with 0xFF reserved.
 *   - Refusal precedence: scale 0xFF, then NaN code, then inexact element;
 *     each reports the lowest row-major index (scale-grid index for 0xFF).
 *   - Ragged edges use a ceil-div grid: element (r,c) takes grid[r/128][c/128].
 *
 * Everything here is written from the format arithmetic (ldexp, frexp) and
 * the plain definitions; none of it is a GPU bit trick.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORC_OK = 0, ORC_ARG = 1, ORC_SCALE_FF = 2, ORC_NAN_CODE = 3, ORC_INEXACT = 4 };

/* O1 [Fp8Dense] (OCP E4M3 reading): value of an e4m3 code byte.
 * Sign = bit 7, exponent field E = bits 6..3, mantissa m = bits 2..0.
 * E == 0: subnormal, m * 2^-9.  E > 0: (8 + m) * 2^(E - 10), i.e. (1 + m/8) * 2^(E-7).
 * E == 15 and m == 7 is NaN: returns 0 and leaves *v alone. */
int orc_e4m3(uint8_t b, double *v)
{
    int sign = b >> 7, E = (b >> 3) & 15, m = b & 7;
    if (E == 15 && m == 7)
        return 0;
    double mag = (E == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    *v = sign ? -mag : mag;
    return 1;
}

/* O2 [Fp8Dense]: value of an e8m0 scale code, 2^(c - 127); 0xFF is refused. */
int orc_e8m0(uint8_t c, double *v)
{
    if (c == 0xFF)
        return 0;
    *v = ldexp(1.0, (int)c - 127);
    return 1;
}

/* bf16 pattern -> double [bf16_to_f32]: the pattern is the high half of an f32. */
double orc_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* O3 [Rungs] bit-level exactness: is v exactly a finite bf16 value?
 * bf16 has 8 significant bits (7 stored), exponents -126..127, subnormals down
 * to 2^-133 and a largest finite value of (2 - 2^-7) * 2^127 = 255 * 2^120.
 * A nonzero v is exact iff |v| <= that maximum and |v| is an integer multiple
 * of the bf16 spacing at its binade, 2^(max(floor(log2|v|), -126) - 7). */
int orc_is_bf16_exact(double v)
{
    if (v == 0.0)
        return 1;
    if (!isfinite(v))
        return 0;
    double a = fabs(v);
    if (a > ldexp(255.0, 120))
        return 0;
    int e;
    frexp(a, &e); /* a = f * 2^e with f in [0.5, 1): floor(log2 a) = e - 1 */
    int binade = e - 1;
    int q = (binade > -126 ? binade : -126) - 7;
    double k = ldexp(a, -q);
    return k == floor(k);
}

/* Exact value of element (r, c): e4m3(code) * e8m0(scale), in double (both
 * factors have at most 4 significant bits, so the product is exact).
 * Returns 0 on a NaN code or a 0xFF scale. */
static int element_value(const uint8_t *codes, const uint8_t *scales, int64_t cols,
                         int64_t r, int64_t c, double *v)
{
    int64_t gc = (cols + 127) / 128;
    double e, s;
    if (!orc_e4m3(codes[r * cols + c], &e))
        return 0;
    if (!orc_e8m0(scales[(r / 128) * gc + c / 128], &s))
        return 0;
    *v = e * s;
    return 1;
}

/* O4 [Fp8Dense], [Rungs]: load-time check and scale-grid decode.
 * Checks, in order: any scale code 0xFF (lowest grid index), any NaN code
 * (lowest element index), any element whose exact value is not a bf16 value
 * (lowest element index). On success writes the f32 grid (2^(c-127) exactly,
 * 2^-127 being an f32 subnormal) and returns ORC_OK. */
int orc_load_check(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                   float *grid_out, int64_t *first_bad)
{
    if (rows < 1 || cols < 1)
        return ORC_ARG;
    int64_t gr = (rows + 127) / 128, gc = (cols + 127) / 128;
    for (int64_t i = 0; i < gr * gc; i++)
        if (scales[i] == 0xFF) {
            *first_bad = i;
            return ORC_SCALE_FF;
        }
    for (int64_t i = 0; i < rows * cols; i++) {
        double v;
        if (!orc_e4m3(codes[i], &v)) {
            *first_bad = i;
            return ORC_NAN_CODE;
        }
    }
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            double v;
            element_value(codes, scales, cols, r, c, &v);
            if (!orc_is_bf16_exact(v)) {
                *first_bad = r * cols + c;
                return ORC_INEXACT;
            }
        }
    for (int64_t i = 0; i < gr * gc; i++) {
        double s;
        orc_e8m0(scales[i], &s);
        grid_out[i] = (float)s;
    }
    *first_bad = -1;
    return ORC_OK;
}

/* O5 [Rungs], [Fp8Dense]: the bf16 dequant slab. Each element's exact value is
 * a bf16 value (checked here), so its f32 image has a zero low half and the
 * bf16 pattern is the high half. Returns ORC_INEXACT (and stops) otherwise. */
int orc_dequant_bf16(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                     uint16_t *out, int64_t *first_bad)
{
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            double v;
            if (!element_value(codes, scales, cols, r, c, &v) || !orc_is_bf16_exact(v)) {
                *first_bad = r * cols + c;
                return ORC_INEXACT;
            }
            float f = (float)v;
            uint32_t bits;
            memcpy(&bits, &f, sizeof bits);
            out[r * cols + c] = (uint16_t)(bits >> 16);
        }
    *first_bad = -1;
    return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* O6 [Rungs], [dense_fp8]: the GEMV in double.
 *   y[m][r]   = sum over c of w(r,c) * x(m,c)
 *   yabs[m][r] = sum over c of |w(r,c) * x(m,c)|
 * with w the exact element value and x the bf16 activation. Every product is
 * exact in double; the sum runs over c in increasing order. Rows are
 * independent, so splitting them over threads changes no result. */

struct gemv64_job {
    const uint8_t *codes, *scales;
    const uint16_t *x;
    int64_t rows, cols, M, r0, r1;
    double *y, *yabs;
};

static void *gemv64_rows(void *p)
{
    struct gemv64_job *j = (struct gemv64_job *)p;
    double e4m3_of[256];
    for (int b = 0; b < 256; b++) {
        double v = NAN;
        orc_e4m3((uint8_t)b, &v);
        e4m3_of[b] = v;
    }
    int64_t gc = (j->cols + 127) / 128;
    for (int64_t m = 0; m < j->M; m++)
        for (int64_t r = j->r0; r < j->r1; r++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t c = 0; c < j->cols; c++) {
                double s;
                orc_e8m0(j->scales[(r / 128) * gc + c / 128], &s);
                double w = e4m3_of[j->codes[r * j->cols + c]] * s;
                double p = w * orc_bf16(j->x[m * j->cols + c]);
                acc += p;
                aacc += fabs(p);
            }
            j->y[m * j->rows + r] = acc;
            j->yabs[m * j->rows + r] = aacc;
        }
    return NULL;
}

void orc_gemv_f64(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                  const uint16_t *x, int64_t M, double *y, double *yabs, int nthreads)
{
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    struct gemv64_job *jobs = (struct gemv64_job *)calloc((size_t)nthreads, sizeof *jobs);
    for (int t = 0; t < nthreads; t++) {
        struct gemv64_job j = {codes, scales, x, rows, cols, M,
                               rows * t / nthreads, rows * (t + 1) / nthreads, y, yabs};
        jobs[t] = j;
        if (t > 0)
            pthread_create(&th[t], NULL, gemv64_rows, &jobs[t]);
    }
    gemv64_rows(&jobs[0]);
    for (int t = 1; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(jobs);
    free(th);
}

/* ------------------------------------------------------------------------- */
/* O7 [Fp8Dense], [batched]: the f32 GEMV in the documented reduction order.
 *
 * The pages fix only that both arms run the same order on the same f32
 * weights. The order used by this library, per output (m, r):
 *   segment t covers columns [1024 t, 1024 t + 1024); within it, lane l
 *   (0..63) owns the 16-column chunk q = 64 t + l, columns [16 q, 16 q + 16).
 *   lane partial  L[l] = fused multiply-add chain over the chunk's 16 columns
 *                 in increasing order, starting from +0.0; a chunk wholly past
 *                 the last column contributes +0.0.
 *   segment sum   P[t] = balanced pairwise tree over the 64 lane partials,
 *                 pairing lanes that differ in bit 5 first, then bit 4, ...,
 *                 bit 0 (L[l] + L[l + h] for h = 32, 16, 8, 4, 2, 1).
 *   output        y = P[0], then y = y + P[t] for t = 1, 2, ... in order.
 * The order depends on cols only: not on rows, on M, on the launch plan or
 * on the device, so row m of a panel equals the single-row result [batched].
 *
 * wsrc selects the weight source:
 *   0 (A): the bf16 dequant slab w_bf16, widened to f32 by placing the 16
 *          bits in the high half [bf16_to_f32];
 *   1 (B): in-register decode, f32(e4m3(code)) * f32(e8m0(scale)) in f32.
 * variant != 0 perturbs the order (used to show that the bitwise identity
 * check can fail): 1 = reverse the 16 columns inside each chunk,
 * 2 = tree pairs lanes in bit 0 first, 3 = sum the segments last to first,
 * 4 = multiply then add (two roundings) in place of the fused multiply-add.
 * Returns ORC_ARG on bad arguments, else ORC_OK. */

#define SEG_COLS 1024
#define LANES 64
#define CHUNK 16

struct gemv32_job {
    int wsrc, variant;
    const uint8_t *codes, *scales;
    const uint16_t *w_bf16, *x;
    int64_t rows, cols, M, r0, r1;
    float *y;
};

static float weight_f32(const struct gemv32_job *j, const float *e4m3_f, int64_t r, int64_t c)
{
    if (j->wsrc == 0) {
        uint32_t bits = (uint32_t)j->w_bf16[r * j->cols + c] << 16;
        float f;
        memcpy(&f, &bits, sizeof f);
        return f;
    }
    int64_t gc = (j->cols + 127) / 128;
    double s;
    orc_e8m0(j->scales[(r / 128) * gc + c / 128], &s);
    float sf = (float)s; /* exact: 2^-127 .. 2^127 are all f32 values */
    return e4m3_f[j->codes[r * j->cols + c]] * sf;
}

static void *gemv32_rows(void *p)
{
    const struct gemv32_job *j = (const struct gemv32_job *)p;
    float e4m3_f[256];
    for (int b = 0; b < 256; b++) {
        double v = NAN;
        orc_e4m3((uint8_t)b, &v);
        e4m3_f[b] = (float)v; /* exact: every finite e4m3 value is an f32 value */
    }
    int64_t T = (j->cols + SEG_COLS - 1) / SEG_COLS;
    float *P = (float *)malloc((size_t)T * sizeof *P);
    for (int64_t m = 0; m < j->M; m++)
        for (int64_t r = j->r0; r < j->r1; r++) {
            for (int64_t t = 0; t < T; t++) {
                float L[LANES];
                for (int l = 0; l < LANES; l++) {
                    int64_t q = LANES * t + l;
                    float a = 0.0f;
                    if (CHUNK * q < j->cols) {
                        for (int jj = 0; jj < CHUNK; jj++) {
                            int k = (j->variant == 1) ? CHUNK - 1 - jj : jj;
                            int64_t c = CHUNK * q + k;
                            float w = weight_f32(j, e4m3_f, r, c);
                            uint32_t xb = (uint32_t)j->x[m * j->cols + c] << 16;
                            float xf;
                            memcpy(&xf, &xb, sizeof xf);
                            if (j->variant == 4) {
                                volatile float prod = w * xf;
                                a = a + prod;
                            } else {
                                a = fmaf(w, xf, a);
                            }
                        }
                    }
                    L[l] = a;
                }
                if (j->variant == 2) {
                    /* bit 0 first: pair (l, l+1), then (l, l+2), ... */
                    for (int h = 1; h < LANES; h *= 2)
                        for (int l = 0; l < LANES; l += 2 * h)
                            L[l] = L[l] + L[l + h];
                } else {
                    for (int h = LANES / 2; h >= 1; h /= 2)
                        for (int l = 0; l < h; l++)
                            L[l] = L[l] + L[l + h];
                }
                P[t] = L[0];
            }
            float acc;
            if (j->variant == 3) {
                acc = P[T - 1];
                for (int64_t t = T - 2; t >= 0; t--)
                    acc = acc + P[t];
            } else {
                acc = P[0];
                for (int64_t t = 1; t < T; t++)
                    acc = acc + P[t];
            }
            j->y[m * j->rows + r] = acc;
        }
    free(P);
    return NULL;
}

int orc_gemv_f32_order(int wsrc, const uint8_t *codes, const uint8_t *scales,
                       const uint16_t *w_bf16, int64_t rows, int64_t cols, const uint16_t *x,
                       int64_t M, int variant, float *y, int nthreads)
{
    if (rows < 1 || cols < 1 || M < 1 || (wsrc != 0 && wsrc != 1) || variant < 0 || variant > 4)
        return ORC_ARG;
    if ((wsrc == 0 && !w_bf16) || (wsrc == 1 && (!codes || !scales)) || !x || !y)
        return ORC_ARG;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    struct gemv32_job *jobs = (struct gemv32_job *)calloc((size_t)nthreads, sizeof *jobs);
    for (int t = 0; t < nthreads; t++) {
        struct gemv32_job jb = {wsrc, variant, codes, scales, w_bf16, x, rows, cols, M,
                                rows * t / nthreads, rows * (t + 1) / nthreads, y};
        jobs[t] = jb;
        if (t > 0)
            pthread_create(&th[t], NULL, gemv32_rows, &jobs[t]);
    }
    gemv32_rows(&jobs[0]);
    for (int t = 1; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return ORC_OK;
}
