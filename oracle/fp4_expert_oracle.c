/*
 * fp4_expert_oracle.c -- plain, slow, obviously correct CPU oracle for the
 * native expert arm: per-128 FP8 activation codes times FP4 (e2m1) weight
 * slabs as stored, in the NVFP4 and MXFP4 recipes.
 *
 * TEST INFRASTRUCTURE. Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load or call this file's library. The
 * product path never does, and this file shares no source with it (nor with
 * fp8blk_oracle.c, apart from being linked into the same test library).
 *
 * Sources (docs.rs pages of the memra-engine crate):
 *   [ExpertArm]  "Module dsv4_gpu" page, enum ExpertArm: the native expert
 *                arm multiplies activation codes quantized per 128 elements
 *                to FP8 by the NVFP4 / MXFP4 expert slabs as stored; the
 *                other arm dequantizes the slab exactly to bf16 and runs a
 *                bf16 GEMM.
 *   [ExpertKind] same page, enum ExpertKind: trunk experts are NVFP4, the
 *                multi-token-prediction experts are MXFP4; the recipe is read
 *                from the stored dtypes and anything unexpected is refused.
 *   [Rungs]      same page, module header (the rungs paragraph): routed NVFP4
 *                experts are dequantized into a bf16 scratch, exactly.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   R1 e2m1 is the OCP FP4 element: sign, 2 exponent bits (bias 1), 1
 *      mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. Two codes per
 *      byte, the even column in the low nibble.
 *   R2 MXFP4: one e8m0 scale 2^(s-127) per 32 consecutive columns of a row;
 *      s = 0xFF is refused.
 *   R3 NVFP4: one e4m3 scale per 16 consecutive columns of a row (OCP E4M3,
 *      as the dense arm's codes); a NaN or negative scale code (sign bit set,
 *      -0 included) is refused. A per-tensor f32 scale multiplies the output
 *      of the GEMV; it is not part of the element value.
 *   R4 act_quant: per row of the activation panel and per block of 128
 *      consecutive columns (the last one may be shorter), the scale is the
 *      smallest power of two 2^e, e in [-127, 127], with amax <= 448 * 2^e;
 *      each code is x / 2^e (exact) rounded to the nearest e4m3 value, ties to
 *      even, keeping the sign of x (so -0 and small negatives give 0x80).
      Parity unpinned as to the choice of scale rule: the pages say only
      that activations become FP8 codes per 128 elements, so nothing on
      them rules out another rule (an f32 scale amax / 448, say). What the
      tests pin is that this routine computes R4 exactly as stated.
 *   R5 the native GEMV: y[m][r] = g * sum over c of q(m, c) * w(r, c), with q
 *      the dequantized activation code and w the element value; the pages fix
 *      no summation order, so the library is checked against this sum by
 *      tolerance.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { FX_OK = 0, FX_ARG = 1, FX_SCALE_FF = 2, FX_INEXACT = 4, FX_BAD_SCALE = 7 };
enum { FX_MXFP4 = 0, FX_NVFP4 = 1 };

/* e4m3 byte -> value (OCP E4M3, as in R3): sign bit 7, exponent field E =
 * bits 6..3 (bias 7), mantissa m = bits 2..0; E == 0 is subnormal m * 2^-9;
 * S.1111.111 is NaN (returns 0). Written again here so this file stands on
 * its own. */
static int fx_e4m3(uint8_t b, double *v)
{
    int E = (b >> 3) & 15, m = b & 7;
    if (E == 15 && m == 7)
        return 0;
    double mag = E == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), E - 10);
    *v = (b & 0x80) ? -mag : mag;
    return 1;
}

static double fx_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Is v exactly a finite bf16 value? (8 significant bits, exponents down to
 * -126 with subnormal spacing 2^-133, largest finite 255 * 2^120.) */
static int fx_is_bf16(double v)
{
    if (v == 0.0)
        return 1;
    if (!isfinite(v) || fabs(v) > ldexp(255.0, 120))
        return 0;
    int e;
    frexp(fabs(v), &e);
    int q = (e - 1 > -126 ? e - 1 : -126) - 7;
    double k = ldexp(fabs(v), -q);
    return k == floor(k);
}

/* O8 [ExpertArm] (R1): value of one e2m1 code (low 4 bits of n). */
double orc_e2m1(int n)
{
    int E = (n >> 1) & 3, m = n & 1;
    double mag = E == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
    return (n & 8) ? -mag : mag;
}

/* The e2m1 code of element (r, c) of a packed slab [rows, cols/2] (R1). */
static int fx_code(const uint8_t *codes, int64_t cols, int64_t r, int64_t c)
{
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? byte >> 4 : byte & 15;
}

static int64_t fx_block(int fmt) { return fmt == FX_MXFP4 ? 32 : 16; }

/* Value of one block-scale code: 2^(s-127) (R2) or e4m3 (R3). Returns 0 for
 * a refused code. */
static int fx_scale(int fmt, uint8_t s, double *v)
{
    if (fmt == FX_MXFP4) {
        if (s == 0xFF)
            return 0;
        *v = ldexp(1.0, (int)s - 127);
        return 1;
    }
    if (s & 0x80)
        return 0;
    return fx_e4m3(s, v);
}

/* O9 [ExpertArm], [ExpertKind] (R1-R3): exact value of element (r, c):
 * e2m1(code) * scale. Both factors have at most 4 significant bits, so the
 * product is exact in double. Returns 0 on a refused scale. */
int orc_fp4_element(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t cols, int64_t r,
                    int64_t c, double *v)
{
    int64_t B = fx_block(fmt);
    double s;
    if (!fx_scale(fmt, scales[r * (cols / B) + c / B], &s))
        return 0;
    *v = orc_e2m1(fx_code(codes, cols, r, c)) * s;
    return 1;
}

static int fx_shape_ok(int fmt, int64_t rows, int64_t cols)
{
    return (fmt == FX_MXFP4 || fmt == FX_NVFP4) && rows >= 1 && cols >= 1 && cols % fx_block(fmt) == 0;
}

/* O10 [ExpertKind], [Rungs]: load-time check of an FP4 slab. In this order:
 *   a refused scale code (MXFP4: 0xFF -> FX_SCALE_FF; NVFP4: NaN or sign bit
 *   set -> FX_BAD_SCALE), lowest index into the scale array [rows, cols/B];
 *   an element whose value is not a finite bf16 value (FX_INEXACT), lowest
 *   row-major element index r * cols + c.
 * Every e2m1 code is a finite value, so the codes themselves are not checked. */
int orc_fp4_load_check(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t rows,
                       int64_t cols, int64_t *first_bad)
{
    *first_bad = -1;
    if (!fx_shape_ok(fmt, rows, cols))
        return FX_ARG;
    int64_t ns = rows * (cols / fx_block(fmt));
    for (int64_t i = 0; i < ns; i++) {
        double v;
        if (!fx_scale(fmt, scales[i], &v)) {
            *first_bad = i;
            return fmt == FX_MXFP4 ? FX_SCALE_FF : FX_BAD_SCALE;
        }
    }
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            double v;
            orc_fp4_element(fmt, codes, scales, cols, r, c, &v);
            if (!fx_is_bf16(v)) {
                *first_bad = r * cols + c;
                return FX_INEXACT;
            }
        }
    return FX_OK;
}

/* O11 [Rungs], [ExpertArm] (the bf16-dequant arm): the bf16 slab [rows, cols]
 * holding every element's exact value (the per-tensor NVFP4 scale is not
 * applied, R3). Stops with FX_INEXACT / a refusal code on the first element
 * that cannot be held exactly. */
int orc_fp4_dequant_bf16(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t rows,
                         int64_t cols, uint16_t *out, int64_t *first_bad)
{
    *first_bad = -1;
    if (!fx_shape_ok(fmt, rows, cols))
        return FX_ARG;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t c = 0; c < cols; c++) {
            double v;
            if (!orc_fp4_element(fmt, codes, scales, cols, r, c, &v) || !fx_is_bf16(v)) {
                *first_bad = r * cols + c;
                return FX_INEXACT;
            }
            float f = (float)v;
            uint32_t bits;
            memcpy(&bits, &f, sizeof bits);
            out[r * cols + c] = (uint16_t)(bits >> 16);
        }
    return FX_OK;
}

/* e4m3 code of the finite value v, which must lie on the e4m3 grid with
 * |v| <= 448: the code whose decoded value equals v, found by search over
 * the 127 non-negative finite codes. */
static uint8_t fx_e4m3_code_of(double v, int negative)
{
    double a = fabs(v);
    for (int b = 0; b < 0x7F; b++) {
        double d;
        if (fx_e4m3((uint8_t)b, &d) && d == a)
            return (uint8_t)(negative ? b | 0x80 : b);
    }
    return 0xFF; /* not reached for values on the grid */
}

/* Round |a| (0 <= a <= 448) to the e4m3 grid, ties to even. The grid spacing
 * is 2^-9 below the smallest normal 2^-6 and 2^(floor(log2 a) - 3) above it;
 * a / spacing is exact in double, so the rounding is decided exactly. */
static double fx_round_e4m3(double a)
{
    double spacing;
    if (a < ldexp(1.0, -6)) {
        spacing = ldexp(1.0, -9);
    } else {
        int e;
        frexp(a, &e); /* a in [2^(e-1), 2^e) */
        spacing = ldexp(1.0, e - 1 - 3);
    }
    double q = a / spacing;
    double n = floor(q);
    double rem = q - n;
    if (rem > 0.5 || (rem == 0.5 && fmod(n, 2.0) == 1.0))
        n += 1.0;
    return n * spacing;
}

/* O12 [ExpertArm] (R4): act_quant. x: bf16 patterns [M, cols]; writes codes
 * [M, cols] and e8m0 scale codes [M, ceil(cols/128)]. x must be finite. */
int orc_act_quant(const uint16_t *x, int64_t M, int64_t cols, uint8_t *codes, uint8_t *scales)
{
    if (M < 1 || cols < 1)
        return FX_ARG;
    int64_t nb = (cols + 127) / 128;
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < nb; b++) {
            int64_t c0 = 128 * b, c1 = c0 + 128 < cols ? c0 + 128 : cols;
            double amax = 0.0;
            for (int64_t c = c0; c < c1; c++) {
                double v = fabs(fx_bf16(x[m * cols + c]));
                if (!isfinite(v))
                    return FX_ARG;
                if (v > amax)
                    amax = v;
            }
            int e = -127;
            while (e < 127 && amax > ldexp(448.0, e))
                e++;
            scales[m * nb + b] = (uint8_t)(e + 127);
            for (int64_t c = c0; c < c1; c++) {
                double v = fx_bf16(x[m * cols + c]);
                double q = fx_round_e4m3(fabs(ldexp(v, -e)));
                codes[m * cols + c] = fx_e4m3_code_of(q, signbit(v) != 0);
            }
        }
    return FX_OK;
}

/* Dequantized activation value q(m, c) = e4m3(code) * 2^(s - 127) (R4). */
static double fx_act_value(const uint8_t *xq, const uint8_t *xs, int64_t cols, int64_t m, int64_t c)
{
    double v = 0.0;
    fx_e4m3(xq[m * cols + c], &v);
    return v * ldexp(1.0, (int)xs[m * ((cols + 127) / 128) + c / 128] - 127);
}

/* O13 [ExpertArm] (R5): the native GEMV in double.
 *   y[m][r]    = g * sum over c of q(m, c) * w(r, c)
 *   yabs[m][r] = |g| * sum over c of |q(m, c) * w(r, c)|
 * Each product q * w is exact in double (at most 4 + 4 significant bits);
 * the sum runs over c in increasing order. Rows are independent, so the
 * split over threads changes no result. */
struct fx_job {
    int fmt;
    const uint8_t *codes, *scales, *xq, *xs;
    double g;
    int64_t rows, cols, M, r0, r1;
    double *y, *yabs;
};

static void *fx_rows(void *p)
{
    const struct fx_job *j = (const struct fx_job *)p;
    for (int64_t m = 0; m < j->M; m++)
        for (int64_t r = j->r0; r < j->r1; r++) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t c = 0; c < j->cols; c++) {
                double w = 0.0;
                orc_fp4_element(j->fmt, j->codes, j->scales, j->cols, r, c, &w);
                double prod = fx_act_value(j->xq, j->xs, j->cols, m, c) * w;
                acc += prod;
                aacc += fabs(prod);
            }
            j->y[m * j->rows + r] = j->g * acc;
            j->yabs[m * j->rows + r] = fabs(j->g) * aacc;
        }
    return NULL;
}

int orc_fp4_gemv_f64(int fmt, const uint8_t *codes, const uint8_t *scales, double g, int64_t rows,
                     int64_t cols, const uint8_t *xq, const uint8_t *xs, int64_t M, double *y,
                     double *yabs, int nthreads)
{
    if (!fx_shape_ok(fmt, rows, cols) || M < 1)
        return FX_ARG;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > rows)
        nthreads = (int)rows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof *th);
    struct fx_job *jobs = (struct fx_job *)calloc((size_t)nthreads, sizeof *jobs);
    for (int t = 0; t < nthreads; t++) {
        struct fx_job jb = {fmt, codes, scales, xq, xs, g, rows, cols, M,
                            rows * t / nthreads, rows * (t + 1) / nthreads, y, yabs};
        jobs[t] = jb;
        if (t > 0)
            pthread_create(&th[t], NULL, fx_rows, &jobs[t]);
    }
    fx_rows(&jobs[0]);
    for (int t = 1; t < nthreads; t++)
        pthread_join(th[t], NULL);
    free(jobs);
    free(th);
    return FX_OK;
}
