/*
 * fp8blk.h -- C ABI of libfp8blk.so: the block-scaled FP8 ("FP8-blk") dense
 * linear, read as stored, on AMD Instinct MI355X (gfx950).
 *
 * The operation (docs.rs pages of the memra-engine crate):
 *   - "Module dsv4_gpu" page, struct Fp8Dense: a linear is held as e4m3
 *     codes [rows, cols] plus a 128x128 grid of e8m0 block scales. Every
 *     scale is a power of two, the grid is decoded to f32 once at load, and
 *     a 0xFF scale is refused there. The GEMV forms e4m3(code) * scale in
 *     registers; that is the same f32 value the bf16 dequant slab holds, and
 *     the accumulation order is the bf16 kernel's, so the two give identical
 *     bits.
 *   - same page, module header (rungs paragraph): dequantization to bf16
 *     refuses any element that is not exactly a bf16 value; activations enter
 *     as bf16; products accumulate in f32.
 *   - same page, enum DW: the GEMV takes raw pointers to either the bf16 slab
 *     or the stored FP8 pair, rebuilt per call by the caller.
 *   - same page, structs StepWs / VerifyWs: work buffers are allocated once
 *     by the owner, never per step; the verify panel is the decode arena
 *     widened to several rows.
 *   - "Struct Dsv4Gpu" page, field dense_fp8: decode and verify read the
 *     FP8-blk linears as stored (e4m3 + f32 block scales) through the twin
 *     GEMVs, halving the dense weight bytes.
 *   - "Struct Dsv4Gpu" page, method spec_greedy_batched_with: a batched
 *     kernel gives the same bits as its single-position twin.
 *   - "dflash.rs" source page, fn bf16_to_f32: a bf16 pattern widens to f32
 *     by becoming the high 16 bits.
 *
 * Formats (this library's reading of the pages' "e4m3" and "e8m0"):
 *   e4m3 = OCP FP8 E4M3: sign bit, 4 exponent bits (bias 7), 3 mantissa bits,
 *          subnormals, no infinities, 0x7F and 0xFF are NaN.
 *   e8m0 = 2^(code - 127); 0xFF is refused.
 *   bf16 = the high 16 bits of an IEEE binary32, passed as uint16_t patterns.
 *
 * Layouts (all row-major and contiguous, no strides):
 *   codes       uint8_t  [rows, cols]  rows = output features, cols = reduction
 *   scales_e8m0 uint8_t  [ceil(rows/128), ceil(cols/128)]; element (r, c) uses
 *                                      entry [r/128][c/128]
 *   scales_f32  float    same grid, as produced by fp8blk_load_check
 *   w_bf16      uint16_t [rows, cols]  bf16 dequant slab
 *   x_bf16      uint16_t [M, cols]     activation panel, M = 1 (decode) .. 16
 *   y           float    [M, rows]
 *
 * Reduction order (fixed; depends on cols only, never on rows, M, the launch
 * plan or the device). For each output (m, r):
 *   - segment t covers columns [1024 t, 1024 t + 1024); lane l = 0..63 owns
 *     the 16-column chunk q = 64 t + l;
 *   - lane partial: fused multiply-add over the chunk's 16 columns in
 *     increasing order, starting from +0.0 (+0.0 for a chunk past the end);
 *   - segment sum: pairwise tree over the 64 lane partials, pairing lanes that
 *     differ in bit 5, then 4, 3, 2, 1, 0;
 *   - y = segment 0, then y += segment t for t = 1, 2, ... in order.
 *   Hence fp8blk_gemv == bf16_gemv_twin bitwise on load-checked weights, row m
 *   of an M-row call == the M = 1 call on x[m] bitwise. Each product w * x is
 *   exact in f32 (at most 4 x 8 significant bits) as long as it stays out of
 *   the f32 subnormal range, so for such inputs the only error is in the sums:
 *   |y - exact| <= gamma_d * sum_c |w x|, d = 16 + 6 + ceil(cols/1024) - 1,
 *   gamma_d = d u / (1 - d u), u = 2^-24; d <= 85 and gamma_d < 5.1e-6 for
 *   every cols up to FP8BLK_MAX_COLS.
 *
 * Ownership and threading: the caller owns every buffer (device memory unless
 * stated). The library allocates and frees nothing, keeps no per-call global
 * state and is safe to call from several host threads. All device work is
 * enqueued on the caller's stream `stream` (NULL = the null stream).
 *
 * Errors: every entry point returns an fp8blk_status. It never aborts, throws
 * or prints. On an error return the outputs are unspecified. fp8blk_dequant_bf16,
 * fp8blk_gemv and bf16_gemv_twin do not re-validate the weights: they assume
 * fp8blk_load_check accepted them (validation happens once, at load).
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* A HIP stream (the same type as hipStream_t). */
typedef struct ihipStream_t *fp8blk_stream_t;

typedef enum fp8blk_status {
    FP8BLK_OK = 0,
    FP8BLK_ERR_ARG = 1,       /* null pointer, bad shape, misalignment, M out of range */
    FP8BLK_ERR_SCALE_FF = 2,  /* a scale code is 0xFF */
    FP8BLK_ERR_NAN_CODE = 3,  /* a weight code is 0x7F or 0xFF (NaN) */
    FP8BLK_ERR_INEXACT = 4,   /* e4m3(code) * scale is not exactly a bf16 value */
    FP8BLK_ERR_WORKSPACE = 5, /* ws is NULL or ws_bytes is below fp8blk_workspace_bytes */
    FP8BLK_ERR_HIP = 6,       /* a HIP launch or runtime call failed */
    FP8BLK_ERR_BAD_SCALE = 7, /* an NVFP4 block scale is negative or NaN */
    FP8BLK_ERR_TIMEOUT = 8    /* a chained launch stopped waiting for an earlier group's outputs */
} fp8blk_status;

/* Operation ids for fp8blk_workspace_bytes. */
typedef enum fp8blk_op {
    FP8BLK_OP_LOAD_CHECK = 0,
    FP8BLK_OP_DEQUANT_BF16 = 1,
    FP8BLK_OP_GEMV = 2,
    FP8BLK_OP_BF16_TWIN = 3,
    FP8BLK_OP_GEMM_STAGED = 4,
    FP8BLK_OP_BF16_GEMM = 5
} fp8blk_op;

/* Shape limits. cols must be a multiple of 16 (one 16-byte code load). */
#define FP8BLK_MIN_COLS 16
#define FP8BLK_MAX_COLS 65536
#define FP8BLK_MAX_M 16
#define FP8BLK_MAX_PANEL 65536 /* rows of a prefill panel (fp8blk_gemm_staged) */

/* Version of this ABI; bumped on any incompatible change. */
int fp8blk_abi_version(void);

/* Static text for a status code. */
const char *fp8blk_strerror(int status);

/* Bytes of device workspace `op` needs for this shape (0 = none; ws may then
 * be NULL). Returns 0 for an unknown op. Pure host function. */
size_t fp8blk_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M);

/*
 * Load-time check and scale-grid decode ("Module dsv4_gpu" page, Fp8Dense and
 * the rungs paragraph). Checks, in this order of precedence:
 *   FP8BLK_ERR_SCALE_FF  some scale code is 0xFF; *first_bad = lowest
 *                        row-major index into the scale grid;
 *   FP8BLK_ERR_NAN_CODE  some code is 0x7F or 0xFF; *first_bad = lowest
 *                        row-major element index r * cols + c;
 *   FP8BLK_ERR_INEXACT   some e4m3(code) * 2^(scale - 127) is not a finite
 *                        bf16 value (too small for bf16's 2^-133 spacing, or
 *                        past its largest finite value); *first_bad as above.
 * On FP8BLK_OK, scales_f32_out holds 2^(code - 127) exactly for every grid
 * entry (2^-127 as an f32 subnormal) and *first_bad = -1.
 *   codes, scales_e8m0, scales_f32_out: device pointers, layouts above;
 *     codes 16-byte aligned, scales_f32_out 4-byte aligned.
 *   rows >= 1; 16 <= cols <= FP8BLK_MAX_COLS; cols % 16 == 0.
 *   ws: device, >= fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK, ...) bytes,
 *     8-byte aligned; its contents on entry do not matter.
 *   first_bad: HOST pointer, may be NULL.
 * Unlike the other entry points this one waits for `stream` to finish before
 * returning, since it returns a verdict.
 */
int fp8blk_load_check(const uint8_t *codes, const uint8_t *scales_e8m0, int64_t rows,
                      int64_t cols, float *scales_f32_out, void *ws, size_t ws_bytes,
                      int64_t *first_bad, fp8blk_stream_t stream);

/*
 * fp8blk_load_check for callers that cannot allocate device memory (a loader
 * running under an allocation-free harness or inside a serving loop that
 * forbids hipMalloc): the same checks, the same statuses, the same first_bad
 * and the same f32 grid, with no ws argument. Its scratch (the three 64-bit
 * verdict slots) is a static 256-byte device array inside the library, one
 * per GPU, held until the process ends; its device address is looked up once
 * per device on the first call there. The call allocates and frees nothing
 * (no hipMalloc, hipFree or allocating library routine) and clears the slots
 * with a kernel before use. Every call on one GPU shares that GPU's array:
 * calls that overlap on the same GPU (several host threads, several
 * streams) race and may return each other's verdicts; serialize them.
 * Arguments, limits, alignment and errors as for fp8blk_load_check, plus
 * FP8BLK_ERR_WORKSPACE if the check would need more than the 256 bytes the
 * array holds (it needs fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK, ...),
 * 256 for every shape today). Waits for `stream` before returning.
 */
int fp8blk_load_check_noalloc(const uint8_t *codes, const uint8_t *scales_e8m0, int64_t rows,
                              int64_t cols, float *scales_f32_out, int64_t *first_bad,
                              fp8blk_stream_t stream);

/*
 * The bf16 dequant slab ("Module dsv4_gpu" page, rungs paragraph and
 * DenseBf16): out_bf16[r, c] = bf16 pattern of e4m3(codes[r, c]) *
 * scales_f32[r/128][c/128]. Exact (no rounding) for weights accepted by
 * fp8blk_load_check; for others the output is unspecified.
 *   codes, out_bf16: device, 16-byte aligned; scales_f32: device, 4-byte aligned.
 *   rows >= 1; 16 <= cols <= FP8BLK_MAX_COLS; cols % 16 == 0.
 * Enqueued on `stream`; does not wait.
 */
int fp8blk_dequant_bf16(const uint8_t *codes, const float *scales_f32, int64_t rows,
                        int64_t cols, uint16_t *out_bf16, fp8blk_stream_t stream);

/*
 * The FP8-blk GEMV, weights read as stored ("Module dsv4_gpu" page, Fp8Dense;
 * "Struct Dsv4Gpu" page, dense_fp8 and spec_greedy_batched_with):
 *   y[m, r] = sum over c of (e4m3(codes[r, c]) * scales_f32[r/128][c/128]) * x[m, c]
 * decoded in registers, f32 accumulation in the reduction order above.
 *   codes, x_bf16: device, 16-byte aligned; scales_f32, y: device, 4-byte aligned.
 *   rows >= 1; 16 <= cols <= FP8BLK_MAX_COLS; cols % 16 == 0; 1 <= M <= FP8BLK_MAX_M.
 *   ws/ws_bytes: fp8blk_workspace_bytes(FP8BLK_OP_GEMV, ...) bytes (currently
 *     0: ws may be NULL).
 * y must not overlap the inputs. Enqueued on `stream`; does not wait.
 */
int fp8blk_gemv(const uint8_t *codes, const float *scales_f32, int64_t rows, int64_t cols,
                const uint16_t *x_bf16, int64_t M, float *y, void *ws, size_t ws_bytes,
                fp8blk_stream_t stream);

/*
 * The bf16-slab twin of fp8blk_gemv ("Module dsv4_gpu" page, Fp8Dense and DW;
 * "dflash.rs" page, bf16_to_f32): the same y, with weights read from the bf16
 * dequant slab and widened to f32, in the same reduction order with the same
 * instructions. On weights accepted by fp8blk_load_check,
 * bf16_gemv_twin(fp8blk_dequant_bf16(codes, scales)) == fp8blk_gemv(codes,
 * scales) bit for bit.
 *   w_bf16, x_bf16: device, 16-byte aligned; y: device, 4-byte aligned.
 *   Shape limits, ws and stream as for fp8blk_gemv.
 */
int bf16_gemv_twin(const uint16_t *w_bf16, int64_t rows, int64_t cols, const uint16_t *x_bf16,
                   int64_t M, float *y, void *ws, size_t ws_bytes, fp8blk_stream_t stream);

/*
 * Grouped launch: several linears that read the same activation panel (the
 * projections of one input, such as q and kv, or gate and up) in one kernel
 * launch. Each output gets exactly the arithmetic of a call of its own, so
 * fp8blk_gemv_grouped({L1, L2}, x) == fp8blk_gemv(L1, x), fp8blk_gemv(L2, x)
 * bit for bit, and likewise for the twin. One launch instead of n removes the
 * fixed per-launch cost; the same idea as the single launch per projection
 * that the device decode path uses for its routed experts ("Module dsv4_gpu",
 * DecodePath).
 *   linears: HOST array of n descriptors, 1 <= n <= FP8BLK_MAX_GROUP; for each,
 *     w = codes (fp8blk_gemv_grouped) or bf16 slab (bf16_gemv_twin_grouped),
 *     scales_f32 = the f32 grid (ignored by the twin), rows >= 1, y = [M, rows].
 *   cols, x_bf16, M: shared by all the linears; limits and alignment as for
 *     fp8blk_gemv. No workspace. Enqueued on `stream`; does not wait.
 */
#define FP8BLK_MAX_GROUP 8
typedef struct fp8blk_linear {
    const void *w;
    const float *scales_f32;
    int64_t rows;
    float *y;
} fp8blk_linear;

int fp8blk_gemv_grouped(const fp8blk_linear *linears, int n, int64_t cols, const uint16_t *x_bf16,
                        int64_t M, fp8blk_stream_t stream);
int bf16_gemv_twin_grouped(const fp8blk_linear *linears, int n, int64_t cols, const uint16_t *x_bf16,
                           int64_t M, fp8blk_stream_t stream);

/*
 * Scaled input: one decode-step linear (or a group of them) whose input is an
 * earlier linear's f32 output, x = bf16(c * src) with the f32 product rounded
 * to nearest even (a NaN product gives the quiet NaN 0x7fc0), formed inside
 * the kernel's activation loads instead of by a separate kernel. This is the
 * step between the dependent launches of the device decode path ("Module
 * dsv4_gpu" page, DecodePath: one launch per projection, each projection
 * reading the previous one's output), the same conversion that
 * fp8blk_gemv_chain applies between its groups. For every output:
 * fp8blk_gemv_scaled_input(L, src, c) == fp8blk_gemv(L, x) and
 * fp8blk_gemv_grouped_scaled_input({L1, ...}, src, c) ==
 * fp8blk_gemv_grouped({L1, ...}, x) bit for bit, with x[k] = bf16(c * src[k])
 * and M = 1.
 *   codes, scales_f32, y / linears: as for fp8blk_gemv / fp8blk_gemv_grouped
 *     (M = 1; y = [rows]).
 *   src_f32: device, 16-byte aligned, cols f32 values; it may be another
 *     linear's y, but not one that this call writes (an overlap with any
 *     output returns FP8BLK_ERR_ARG).
 *   c: any f32 (the caller's scale).
 *   cols: as for fp8blk_gemv, and at most 16 * 1024 (the single-row kernel's
 *     range); larger cols return FP8BLK_ERR_ARG.
 * No workspace. Enqueued on `stream`; does not wait.
 */
int fp8blk_gemv_scaled_input(const uint8_t *codes, const float *scales_f32, int64_t rows, int64_t cols,
                             const float *src_f32, float c, float *y, fp8blk_stream_t stream);
int fp8blk_gemv_grouped_scaled_input(const fp8blk_linear *linears, int n, int64_t cols, const float *src_f32,
                                     float c, fp8blk_stream_t stream);

/*
 * Next input: the same step done by the producer instead. One activation row
 * (M = 1); besides its f32 output the linear (for the grouped form, linear k
 * of the group) writes x_next[r] = bf16(c * y[r]), the f32 product rounded to
 * nearest even (a NaN gives 0x7fc0), the bf16 input of the dependent linear
 * that follows ("Module dsv4_gpu" page, DecodePath). y is exactly
 * fp8blk_gemv's (fp8blk_gemv_grouped's) and x_next is exactly what
 * fp8blk_gemv_scaled_input forms from y, so a chain of these launches gives
 * every output bit for bit as separate launches with the conversion between
 * them.
 *   codes, scales_f32, x_bf16, y / linears: as for fp8blk_gemv /
 *     fp8blk_gemv_grouped with M = 1; cols at most 16 * 1024 (else
 *     FP8BLK_ERR_ARG).
 *   k: 0 <= k < n, the linear whose output feeds x_next.
 *   c: any f32. x_next: device, 2-byte aligned, rows (of linear k) bf16
 *     values; an overlap with x_bf16 or any output returns FP8BLK_ERR_ARG.
 * No workspace. Enqueued on `stream`; does not wait.
 */
int fp8blk_gemv_next_input(const uint8_t *codes, const float *scales_f32, int64_t rows, int64_t cols,
                           const uint16_t *x_bf16, float *y, float c, uint16_t *x_next, fp8blk_stream_t stream);
int fp8blk_gemv_grouped_next_input(const fp8blk_linear *linears, int n, int64_t cols, const uint16_t *x_bf16,
                                   int k, float c, uint16_t *x_next, fp8blk_stream_t stream);

/*
 * Matrix-core arm ("Module dsv4_gpu" page, Fp8Dense; "Struct Dsv4Gpu" page,
 * dense_fp8 and spec_greedy_batched_with). The same y as fp8blk_gemv, with the
 * products run on gfx950's matrix cores (v_mfma_f32_16x16x32_bf16): the
 * weights are decoded in registers to the bf16 values the dequant slab holds
 * and the activation panel is consumed as bf16, padded to 16 rows, so the
 * call stays bound by HBM for every M <= 16.
 *   - fp8blk_gemv_mfma == bf16_gemv_twin_mfma(fp8blk_dequant_bf16(...)) bit for
 *     bit on load-checked weights (same instruction sequence, same operands);
 *   - row m of an M-row call == the 1-row call on x[m], bit for bit;
 *   - the matrix core adds the 32 products of an instruction in an order the
 *     hardware does not document, so the bits differ from fp8blk_gemv's
 *     documented order; the result is within 1e-5 * sum_c |w x| of the exact
 *     sum for every weight the load check accepts, bf16-subnormal weights and
 *     activations included (gfx950's matrix core keeps bf16 subnormal
 *     operands and f32 subnormal sums; tested at scale codes 0..9 and
 *     238..246, on the subnormal e4m3 codes and on subnormal activations).
 * Column order: windows of 128 columns (one scale-block column) in increasing
 * order; in window w, lane group kg (0..3) feeds the 8 columns starting at
 * 128 w + 32 kg + 16 u + 8 v to instruction (u, v) = (0,0), (0,1), (1,0),
 * (1,1), all four into the same f32 accumulator. A row's windows may be split
 * into 2, 4 or 8 contiguous parts, as a function of (rows, cols) only (the
 * largest split that leaves at least 8 windows per part, or at least 4 while
 * fewer than 1024 single-tile waves would run), whose partial sums are added
 * in part order.
 * Arguments, limits, alignment, ownership and stream as for fp8blk_gemv /
 * bf16_gemv_twin; no workspace. Enqueued on `stream`; does not wait.
 */
int fp8blk_gemv_mfma(const uint8_t *codes, const float *scales_f32, int64_t rows, int64_t cols,
                     const uint16_t *x_bf16, int64_t M, float *y, fp8blk_stream_t stream);
int bf16_gemv_twin_mfma(const uint16_t *w_bf16, int64_t rows, int64_t cols, const uint16_t *x_bf16,
                        int64_t M, float *y, fp8blk_stream_t stream);

/*
 * Sequence launch: a list of independent linears, each with its own weights,
 * activation panel and output (for example every dense projection of a
 * decode step, read as stored: "Struct Dsv4Gpu" page, field dense_fp8; or of a
 * verify step, whose panel holds the T <= 16 positions: same page,
 * spec_greedy_batched_with), run by one persistent kernel. The weights of the
 * next linears are already being read while the current ones finish, so HBM
 * stays busy across the whole list instead of ramping up and draining once
 * per linear.
 *
 * Arms (the `arm` of fp8blk_sequence_init and the launch that runs it):
 *   FP8BLK_ARM_FP8 / FP8BLK_ARM_BF16 -> fp8blk_gemv_sequence /
 *     bf16_gemv_twin_sequence: M = 1; each y_j == fp8blk_gemv (resp.
 *     bf16_gemv_twin) of linear j, bit for bit (the documented order above).
 *   FP8BLK_ARM_FP8_MFMA / FP8BLK_ARM_BF16_MFMA -> fp8blk_gemv_mfma_sequence /
 *     bf16_gemv_twin_mfma_sequence: 1 <= M <= 16, the same M for every linear;
 *     the matrix-core arm's arithmetic with the columns of a row taken in one
 *     part (its 128-column windows in increasing order, all into one
 *     accumulator): equal bit for bit to fp8blk_gemv_mfma wherever that call
 *     splits a row into one part, within its tolerance otherwise; the FP8 and
 *     bf16 arms give identical bits, and row m of the panel equals the M = 1
 *     sequence on x[m], bit for bit.
 *
 * The list must be independent: no linear's y may overlap any linear's w,
 * scales_f32 or x_bf16, nor another linear's y. A chain in which one linear
 * consumes another's output needs one launch (or sequence) per link.
 *
 * Two steps, in the spirit of the pages' work buffers that are set up once by
 * their owner ("Module dsv4_gpu" page, StepWs):
 *   fp8blk_sequence_init   validates the n descriptors (HOST array), writes a
 *                          plan of fp8blk_sequence_bytes(n) bytes into the
 *                          caller's device buffer ws (64-byte aligned), and
 *                          fills the HOST struct *seq. It copies the plan to
 *                          the device on `stream` and waits for that copy.
 *                          The plan holds the pointers: the buffers must stay
 *                          allocated, at the same addresses, while seq is used.
 *   the launch             the whole list on `stream`. The vector arms run one
 *                          persistent launch over the full steps of every
 *                          linear whose cols is 1024, 2048 or a multiple of
 *                          4096, and a second one, only if needed, for the
 *                          rest (a last group of rows, linears of other cols);
 *                          the matrix-core arms one launch. Enqueued on
 *                          `stream`; does not wait; may be captured in a HIP
 *                          graph. ws must not be changed meanwhile.
 * Per linear: w = codes (FP8 arms) or bf16 slab (twin arms), scales_f32 = the
 * f32 grid (FP8 arms; ignored by the twin arms), rows >= 1, cols as for
 * fp8blk_gemv, M as above, x_bf16 = [M, cols], y = [M, rows]; alignment as for
 * fp8blk_gemv. 1 <= n <= FP8BLK_MAX_SEQ. Errors: FP8BLK_ERR_ARG (bad
 * descriptor, arm, M or seq; a launch whose arm differs from the plan's),
 * FP8BLK_ERR_WORKSPACE (ws NULL, misaligned or too small), FP8BLK_ERR_HIP.
 */
#define FP8BLK_MAX_SEQ 65536
#define FP8BLK_ARM_FP8 0
#define FP8BLK_ARM_BF16 1
#define FP8BLK_ARM_FP8_MFMA 2
#define FP8BLK_ARM_BF16_MFMA 3
typedef struct fp8blk_seq_linear {
    const void *w;
    const float *scales_f32;
    int64_t rows;
    int64_t cols;
    int64_t M;
    const uint16_t *x_bf16;
    float *y;
} fp8blk_seq_linear;

typedef struct fp8blk_sequence {
    const void *plan;      /* device: the plan inside ws */
    int64_t units_dense;   /* work units of the first launch */
    int64_t units_general; /* work units of the second launch (vector arms: ragged rows or cols) */
    int32_t n;             /* linears */
    int32_t arm;           /* FP8BLK_ARM_* */
    int32_t grid_dense;    /* workgroups of each launch (from the device's compute units, the arm and M) */
    int32_t grid_general;
    int32_t M;             /* panel rows (1 for the vector arms) */
    int32_t reserved;
} fp8blk_sequence;

size_t fp8blk_sequence_bytes(int n);
int fp8blk_sequence_init(fp8blk_sequence *seq, int arm, const fp8blk_seq_linear *linears, int n,
                         void *ws, size_t ws_bytes, fp8blk_stream_t stream);
int fp8blk_gemv_sequence(const fp8blk_sequence *seq, fp8blk_stream_t stream);
int bf16_gemv_twin_sequence(const fp8blk_sequence *seq, fp8blk_stream_t stream);
int fp8blk_gemv_mfma_sequence(const fp8blk_sequence *seq, fp8blk_stream_t stream);
int bf16_gemv_twin_mfma_sequence(const fp8blk_sequence *seq, fp8blk_stream_t stream);

/*
 * Chained launch: the projections of a decode step that feed one another
 * ("Module dsv4_gpu" page, DecodePath: one launch per projection, each reading
 * what the one before it wrote), as ONE persistent launch instead of one
 * launch per link.
 *
 * The list is n_linears FP8-blk linears (fp8blk_linear: w = codes, scales_f32
 * = the f32 grid, rows, y = [rows] f32; M = 1) in n_groups groups, in order.
 * Group g is linears [first, first + n) (the groups tile the list in order),
 * all with `cols` columns (1024, 2048, 3072 or 4096) and one input:
 *   src = -1: the chain input x0_bf16 [cols] (bf16 bits, 16-byte aligned);
 *   src >= 0: the output of linear `src` of an EARLIER group (its rows ==
 *             cols), as x[c] = bf16(c_g * y_src[c]) -- the f32 product c_g *
 *             y (one rounding) rounded to bf16 to nearest even (NaN: 0x7FC0).
 *             The scale stands in for the elementwise work an engine does
 *             between two projections; norms, attention and activations are
 *             not part of this library.
 * Every y_j is written, and equals fp8blk_gemv(w_j, scales_j, x_g) on that
 * group's input bit for bit (the documented order of fp8blk_gemv).
 *
 *   fp8blk_chain_bytes  workspace bytes for this list (0: the list is
 *                       invalid): descriptors, control words, and one 8-byte
 *                       word per output row of every linear that is a src.
 *   fp8blk_chain_init   validates the HOST arrays, writes the plan into the
 *                       caller's device buffer ws (256-byte aligned, at least
 *                       fp8blk_chain_bytes), zeroes its control words, fills
 *                       the HOST struct *ch, and waits for `stream`. The plan
 *                       holds the pointers: the buffers must stay allocated,
 *                       at the same addresses, while ch is used.
 *   fp8blk_gemv_chain   enqueues the whole list as one cooperative launch
 *                       (one workgroup per compute unit, every workgroup
 *                       resident at once) on `stream`; does not wait. The
 *                       outputs of linears that feed later groups are handed
 *                       on through ws, not through a kernel boundary: ws and
 *                       the chain's y buffers must not be touched by other
 *                       work until it completes, and two chained launches on
 *                       one ws must not overlap (calls in stream order are
 *                       fine, any number of times; not capturable in a HIP
 *                       graph).
 *   fp8blk_chain_status waits for `stream`, then returns FP8BLK_OK, or
 *                       FP8BLK_ERR_TIMEOUT if a launch since the last check
 *                       stopped waiting for an input (every wait is bounded,
 *                       seconds; the outputs are then unspecified), and
 *                       clears the record.
 * Errors: FP8BLK_ERR_ARG (a bad list, struct or x0), FP8BLK_ERR_WORKSPACE (ws
 * NULL, misaligned or too small), FP8BLK_ERR_HIP (including a device that
 * cannot hold one workgroup per compute unit at once).
 */
#define FP8BLK_MAX_CHAIN 65536
typedef struct fp8blk_chain_group {
    int32_t first; /* the group's first linear */
    int32_t n;     /* its linears, >= 1 */
    int64_t cols;  /* shared by its linears */
    int32_t src;   /* -1: x0; else the linear whose output is the input */
    float c;       /* input scale (src >= 0) */
} fp8blk_chain_group;

typedef struct fp8blk_chain {
    void *plan;        /* device: the plan inside ws */
    int64_t units;     /* work units (8 chunk slots of one linear) over the list */
    int32_t n_linears;
    int32_t n_groups;
    int32_t grid;      /* workgroups: the device's compute units */
    int32_t reserved;
} fp8blk_chain;

size_t fp8blk_chain_bytes(const fp8blk_linear *linears, int n_linears, const fp8blk_chain_group *groups,
                          int n_groups);
int fp8blk_chain_init(fp8blk_chain *ch, const fp8blk_linear *linears, int n_linears,
                      const fp8blk_chain_group *groups, int n_groups, void *ws, size_t ws_bytes,
                      fp8blk_stream_t stream);
int fp8blk_gemv_chain(const fp8blk_chain *ch, const uint16_t *x0_bf16, fp8blk_stream_t stream);
int fp8blk_chain_status(const fp8blk_chain *ch, fp8blk_stream_t stream);

/*
 * Staged prefill GEMM ("Module dsv4_gpu" page, rungs paragraph and
 * DenseBf16: under the FP8 arm, prefill stages the dense weights as a
 * transient bf16 copy and runs the bf16 GEMM over it). For a prefill panel of
 * N tokens:
 *   y[n, r] = sum over c of slab[r, c] * x[n, c],  slab = fp8blk_dequant_bf16(codes, scales)
 * fp8blk_gemm_staged writes the slab into the first part of ws (exact, as
 * fp8blk_dequant_bf16) and then runs one hipBLASLt bf16 x bf16 -> f32 GEMM
 * (f32 accumulation) over it; bf16_gemm_twin runs the same GEMM over a slab
 * the caller holds. On weights accepted by fp8blk_load_check the two give
 * identical bits (the same GEMM on the same values). The GEMM's summation
 * order is the library's: every product is exact in f32 (bf16 x bf16), so
 * |y - exact| <= gamma_cols * sum_c |w x| (gamma_k = k u / (1 - k u),
 * u = 2^-24) whatever the order; the typical error is far smaller.
 *   codes, w_bf16, x_bf16 [N, cols], y [N, rows]: device, 16-byte aligned;
 *   scales_f32: device, 4-byte aligned; shape limits as for fp8blk_gemv;
 *   1 <= N <= FP8BLK_MAX_PANEL.
 *   ws: device, 256-byte aligned, >= fp8blk_workspace_bytes(FP8BLK_OP_GEMM_STAGED
 *     or FP8BLK_OP_BF16_GEMM, rows, cols, N) bytes: the slab (staged only)
 *     plus 32 MB for the library GEMM.
 * The library keeps one hipBLASLt handle per device and the algorithm chosen
 * for each shape (device, rows, cols, N), for the life of the process (host
 * state; no device memory). The first call of a shape, staged or twin, times
 * the library's best 64 heuristic candidates on `stream` (each given a 32 MB
 * workspace, whatever ws_bytes holds beyond that) and keeps the fastest: that
 * call waits for the stream, and it may not be made under graph capture
 * (FP8BLK_ERR_ARG). Every later call of the shape, either entry point,
 * captured or not, runs that algorithm, so the staged call and the twin give
 * identical bits within a process; another process may time a different
 * algorithm and so give other bits, within the same bound. Later calls are
 * enqueued on `stream` and do not wait. Errors: FP8BLK_ERR_ARG,
 * FP8BLK_ERR_WORKSPACE, FP8BLK_ERR_HIP (also when the library has no
 * algorithm for the shape).
 */
int fp8blk_gemm_staged(const uint8_t *codes, const float *scales_f32, int64_t rows, int64_t cols,
                       const uint16_t *x_bf16, int64_t N, float *y, void *ws, size_t ws_bytes,
                       fp8blk_stream_t stream);
int bf16_gemm_twin(const uint16_t *w_bf16, int64_t rows, int64_t cols, const uint16_t *x_bf16, int64_t N,
                   float *y, void *ws, size_t ws_bytes, fp8blk_stream_t stream);

/*
 * Native expert arm ("Module dsv4_gpu" page, enums ExpertArm and ExpertKind,
 * and the rungs paragraph). Routed experts keep their FP4 weight slabs as
 * stored; the activation is quantized to FP8 codes per 128 elements, and the
 * GEMV multiplies the dequantized codes on gfx950's bf16 matrix instruction
 * (v_mfma_f32_16x16x32_bf16, f32 accumulation): both operands are decoded in
 * registers to their exact values, which are bf16 values. (gfx950's scaled
 * FP8 x FP4 instruction was measured to keep only about 13 bits below the
 * largest product of each instruction, about 1e-4 of sum |q w| on random
 * codes, so it is not used.) The bf16-dequant arm, the pages' fallback and
 * A/B reference, is fp4_dequant_bf16 followed by bf16_gemv_twin.
 *
 * Formats (this library's reading; the pages name the recipes only):
 *   e2m1     OCP FP4: sign, 2 exponent bits (bias 1), 1 mantissa bit; values
 *            +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}; two per byte, the even column in
 *            the low nibble.
 *   MXFP4    (FP8BLK_FMT_MXFP4) one e8m0 scale 2^(s-127) per 32 consecutive
 *            columns of a row; 0xFF is refused.
 *   NVFP4    (FP8BLK_FMT_NVFP4) one e4m3 scale per 16 consecutive columns of
 *            a row (non-negative and finite, else refused), plus one f32
 *            per-tensor scale that multiplies the GEMV output.
 *   act_quant per row of the activation and per 128 columns: the scale is
 *            2^e, the smallest power of two with e in [-127, 127] and
 *            amax <= 448 * 2^e (its e8m0 code e + 127 is stored); each code
 *            is the e4m3 value nearest to x / 2^e, ties to even, with the
 *            sign of x.
 *
 * Layouts (row-major, contiguous):
 *   codes        uint8 [rows, cols/2]    packed e2m1
 *   scales       uint8 [rows, cols/32] (MXFP4) or [rows, cols/16] (NVFP4)
 *   xq           uint8 [M, cols]         e4m3 activation codes
 *   xs           uint8 [M, ceil(cols/128)] e8m0 activation scale codes
 *   w_bf16       uint16 [rows, cols]     bf16 slab (the dequant arm)
 *   y            float [M, rows]
 */
#define FP8BLK_FMT_MXFP4 0
#define FP8BLK_FMT_NVFP4 1
#define FP8BLK_ARM_MXFP4 4
#define FP8BLK_ARM_NVFP4 5

/*
 * act_quant as above: x_bf16 [M, cols] -> xq [M, cols], xs [M, ceil(cols/128)].
 * The last block may be shorter than 128 columns. x must be finite (a block
 * holding an infinity or NaN gives unspecified codes).
 *   x_bf16, xq: device, 16-byte aligned; xs: device.
 *   1 <= M <= FP8BLK_MAX_M; 16 <= cols <= FP8BLK_MAX_COLS; cols % 16 == 0.
 * Bit-exact: every code and scale is decided in integer arithmetic.
 * Enqueued on `stream`; does not wait.
 */
int fp8blk_act_quant(const uint16_t *x_bf16, int64_t M, int64_t cols, uint8_t *xq, uint8_t *xs,
                     fp8blk_stream_t stream);

/*
 * Load-time check of an FP4 expert slab ("Module dsv4_gpu" page, ExpertKind:
 * an unexpected recipe is refused). In this order of precedence:
 *   FP8BLK_ERR_SCALE_FF   (MXFP4) a scale code is 0xFF;
 *   FP8BLK_ERR_BAD_SCALE  (NVFP4) a scale code is negative (sign bit set, -0
 *                         included) or NaN;
 *                         *first_bad = lowest index into the scale array;
 *   FP8BLK_ERR_INEXACT    (MXFP4) an element e2m1 * 2^(s-127) is past bf16's
 *                         largest finite value (scale codes 253 and 254);
 *                         *first_bad = lowest element index r * cols + c.
 * Every e2m1 code is finite and every NVFP4 element is a bf16 value, so
 * nothing else is refused.
 *   codes: device, 16-byte aligned; scales: device.
 *   rows >= 1; 32 <= cols <= FP8BLK_MAX_COLS; cols % 32 == 0.
 *   ws: device, 8-byte aligned, >= fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK,
 *     ...) bytes. first_bad: HOST pointer, may be NULL.
 * Waits for `stream` before returning (it returns a verdict).
 */
int fp4_load_check(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                   void *ws, size_t ws_bytes, int64_t *first_bad, fp8blk_stream_t stream);

/*
 * The bf16-dequant arm's slab ("Module dsv4_gpu" page, rungs paragraph:
 * routed experts dequantize exactly into a bf16 scratch; ExpertArm
 * Bf16Dequant): out_bf16[r, c] = e2m1(code) * block scale, exact for slabs
 * accepted by fp4_load_check. NVFP4's per-tensor scale is not applied (it
 * multiplies the GEMV output). Then bf16_gemv_twin(out_bf16, x) * global
 * scale is that arm's GEMV.
 *   codes, out_bf16: device, 16-byte aligned; scales: device (NVFP4: 2-byte
 *   aligned). Shape as for fp4_load_check. Enqueued on `stream`.
 */
int fp4_dequant_bf16(int fmt, const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t cols,
                     uint16_t *out_bf16, fp8blk_stream_t stream);

/*
 * The native expert GEMV ("Module dsv4_gpu" page, ExpertArm Native):
 *   y[m, r] = g * sum over c of q(m, c) * w(r, c)
 * with q = e4m3(xq[m, c]) * 2^(xs[m][c/128] - 127), w = e2m1(code) * block
 * scale and g = global_scale (NVFP4's per-tensor scale; pass 1 for MXFP4).
 * Every product is exact. Order: for each output, the 32-column blocks in
 * increasing order; MXFP4: each block's 32 products are summed by one matrix
 * instruction into the f32 accumulator; NVFP4: the instruction sums each
 * 16-column block, and the sum times its e4m3 scale is added (one fused
 * multiply-add) into one of four f32 accumulators B(p, j), p the block's
 * parity inside its 32-column block k and j = k mod 2 (128 columns at a
 * time, k = j before k = j + 2); the output is
 * g * ((B(0,0) + B(0,1)) + (B(1,0) + B(1,1))). Hence
 * |y - exact| <= gamma_d * |g| * sum_c |q w|, d = 33 + cols / 32
 * (gamma_d = d u / (1 - d u), u = 2^-24; below 1e-5 for cols <= 4096),
 * assuming the instruction's sum of 32 products is no worse than 32 f32
 * additions (measured), while every partial sum stays in f32's range. The
 * conversions and the matrix instruction keep bf16 subnormal operands and f32
 * subnormal sums (tested at MXFP4 scale codes 0..6 and NVFP4's subnormal
 * e4m3 scales).
 *   codes, xq: device, 16-byte aligned; scales: device, 4-byte (MXFP4) or
 *   8-byte (NVFP4) aligned; xs: device; y: device, 4-byte aligned.
 *   rows >= 1; 128 <= cols <= FP8BLK_MAX_COLS; cols % 128 == 0;
 *   1 <= M <= FP8BLK_MAX_M; global_scale finite.
 * Row m of an M-row call equals the 1-row call on row m, bit for bit.
 * y must not overlap the inputs. Enqueued on `stream`; does not wait.
 */
int fp4_expert_gemv(int fmt, const uint8_t *codes, const uint8_t *scales, float global_scale, int64_t rows,
                    int64_t cols, const uint8_t *xq, const uint8_t *xs, int64_t M, float *y,
                    fp8blk_stream_t stream);

/*
 * One launch per projection over the activated experts ("Module dsv4_gpu"
 * page, DecodePath: the device path dispatches the routed experts of a
 * projection in one launch): a list of independent expert linears of one
 * format, each with its own slab, activation codes and output, run by one
 * persistent kernel; y_j is fp4_expert_gemv of linear j, bit for bit.
 * fp4_expert_sequence_init validates the n descriptors (HOST array), writes a
 * plan of fp8blk_sequence_bytes(n) bytes into the device buffer ws (64-byte
 * aligned) and fills *seq (arm FP8BLK_ARM_MXFP4 or FP8BLK_ARM_NVFP4); it
 * copies the plan on `stream` and waits for the copy. The buffers must stay
 * at the same addresses while seq is used. Every linear takes the same M;
 * limits and alignment per linear as for fp4_expert_gemv; no linear's y may
 * overlap any input or another y. fp4_expert_sequence enqueues the list on
 * `stream` (may be captured in a HIP graph). Errors as for
 * fp8blk_sequence_init.
 */
typedef struct fp4_expert_linear {
    const uint8_t *codes;
    const uint8_t *scales;
    float global_scale;
    int64_t rows;
    int64_t cols;
    int64_t M;
    const uint8_t *xq;
    const uint8_t *xs;
    float *y;
} fp4_expert_linear;

int fp4_expert_sequence_init(fp8blk_sequence *seq, int fmt, const fp4_expert_linear *linears, int n,
                             void *ws, size_t ws_bytes, fp8blk_stream_t stream);
int fp4_expert_sequence(const fp8blk_sequence *seq, fp8blk_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
