// Native expert arm: activations quantized to FP8 per 128 elements times FP4
// (e2m1) expert slabs as stored, in the MXFP4 and NVFP4 recipes, plus the
// bf16-dequant arm's exact slab.
//
// "Module dsv4_gpu" page (memra-engine docs): enum ExpertArm (the native arm
// multiplies per-128 FP8 activation codes by the NVFP4 / MXFP4 slabs as
// stored; the other arm dequantizes exactly to bf16 and runs a bf16 GEMM),
// enum ExpertKind (trunk experts NVFP4, multi-token-prediction experts MXFP4,
// anything unexpected refused), the rungs paragraph (routed experts
// dequantize exactly into a bf16 scratch) and enum DecodePath (the routed
// experts of a projection go out in one launch).
//
// The GEMV decodes both operands in registers to exact bf16 values and runs
// on the bf16 matrix instruction with f32 accumulation (see "The native
// GEMV" below). gfx950 also has a scaled FP8 x FP4 matrix instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4); measured on random codes, it keeps
// only about 13 bits below the largest product of each instruction (errors
// near 1e-4 of sum |q w|), so it is not used.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <vector>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMX = FP8BLK_FMT_MXFP4, kNV = FP8BLK_FMT_NVFP4;
constexpr int kActBlock = 128;   // activation scale block (columns)
constexpr int kStepCols = 128;   // columns per matrix instruction
constexpr int kTileRows = 16;    // weight rows per matrix instruction
constexpr int kExWaveLdsBytes = 80 * 1024 / 4;  // LDS of one wave of the native GEMV (a quarter of a workgroup's)
constexpr unsigned long long kNone = ~0ull;

inline int fp4_block(int fmt) { return fmt == kMX ? 32 : 16; }

// ---------------------------------------------------------------------------
// act_quant

// Exponent e of a block's scale 2^e from the bf16 pattern a of its largest
// magnitude, a = f * 2^E with f in [1, 2): amax <= 448 * 2^e = 1.75 * 2^(8+e)
// holds iff E <= 8 + e when f <= 1.75 (mantissa field <= 96), else iff
// E <= 7 + e. A zero or bf16-subnormal amax is below 448 * 2^-127.
__device__ __forceinline__ int act_exp(uint32_t a) {
    const int E = (int)(a >> 7);
    if (E == 0) return -127;
    const int e = E - 135 + ((a & 0x7Fu) > 96u ? 1 : 0);
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// e4m3 code nearest to h * 2^-e (h a bf16 pattern), ties to even, sign kept,
// in integer arithmetic. The magnitude is sig * 2^X with sig at most 8 bits;
// e4m3 steps by 2^(p-3) in the binade [2^p, 2^(p+1)) for p >= -6 and by 2^-9
// below 2^-6; n counts steps, and for a normal result the code is the binade's
// first code plus n - 8 (a carry into the next binade lands on its first
// code). The caller guarantees |h| * 2^-e <= 448.
__device__ __forceinline__ uint32_t act_code(uint32_t h, int e) {
    const uint32_t sign = (h >> 8) & 0x80u;
    const uint32_t E = (h >> 7) & 0xFFu, m = h & 0x7Fu;
    const uint32_t sig = E ? (0x80u | m) : m;
    if (sig == 0) return sign;
    const int X = (E ? (int)E : 1) - 134 - e;
    const int p = X + (31 - __clz(sig));
    const int t = p >= -6 ? p - 3 : -9;
    const int sh = t - X;
    uint32_t n;
    if (sh <= 0) {
        n = sig << -sh;
    } else if (sh >= 9) {
        n = 0;  // sig < 2^8: below half a step
    } else {
        n = sig >> sh;
        const uint32_t rem = sig & ((1u << sh) - 1u), half = 1u << (sh - 1);
        if (rem > half || (rem == half && (n & 1u))) ++n;
    }
    return sign | (p >= -6 ? (uint32_t)((p + 7) << 3) + n - 8u : n);
}

// One wave per (row of the panel, 128-column block); two columns per lane.
__global__ __launch_bounds__(kLanes) void k_act_quant(const uint16_t* __restrict__ x, int64_t cols, int nb,
                                                      uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
    const int b = blockIdx.x, m = blockIdx.y, lane = threadIdx.x;
    const int64_t c = (int64_t)b * kActBlock + 2 * lane;
    const bool in = c < cols;  // cols is even: both columns or neither
    uint32_t d = 0;
    if (in) d = *reinterpret_cast<const uint32_t*>(x + (int64_t)m * cols + c);
    uint32_t a = max(d & 0x7FFFu, (d >> 16) & 0x7FFFu);  // magnitudes order as their patterns
    for (int h = 32; h >= 1; h >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, h));
    const int e = act_exp(a);
    if (in) {
        const uint32_t lo = act_code(d & 0xFFFFu, e), hi = act_code(d >> 16, e);
        *reinterpret_cast<uint16_t*>(xq + (int64_t)m * cols + c) = (uint16_t)(lo | (hi << 8));
    }
    if (lane == 0) xs[(int64_t)m * nb + b] = (uint8_t)(e + 127);
}

// ---------------------------------------------------------------------------
// Load check and the bf16 slab

__global__ void k_fp4_verdict_init(unsigned long long* v) {
    if (threadIdx.x < 3) v[threadIdx.x] = kNone;
}

// One thread per block scale. verdict[0]: lowest MXFP4 scale 0xFF;
// verdict[1]: lowest NVFP4 scale that is negative or NaN; verdict[2]: lowest
// element index of an MXFP4 value past bf16's largest finite value
// (255 * 2^120 ~ 1.99 * 2^127): with scale 2^126 (code 253) the magnitudes 4
// and 6 overflow, with 2^127 (code 254) also 2 and 3, i.e. magnitude fields
// >= 6 and >= 4.
template <int FMT>
__global__ void k_fp4_check(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t rows,
                            int64_t cols, unsigned long long* __restrict__ verdict) {
    constexpr int B = FMT == kMX ? 32 : 16;
    const int64_t per_row = cols / B, n = rows * per_row;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t s = scales[i];
        if constexpr (FMT == kNV) {
            if ((s & 0x80u) || s == 0x7Fu) atomicMin(&verdict[1], (unsigned long long)i);
        } else {
            if (s == 0xFFu) {
                atomicMin(&verdict[0], (unsigned long long)i);
            } else if (s >= 253u) {
                const uint32_t lim = s == 253u ? 6u : 4u;
                const int64_t r = i / per_row, c0 = (i - r * per_row) * B;
                const uint8_t* p = codes + r * (cols / 2) + c0 / 2;
                for (int k = 0; k < B; ++k) {
                    const uint32_t nib = (p[k >> 1] >> (4 * (k & 1))) & 15u;
                    if ((nib & 7u) >= lim) {
                        atomicMin(&verdict[2], (unsigned long long)(r * cols + c0 + k));
                        break;
                    }
                }
            }
        }
    }
}

// e4m3 scale bytes 0 and 1 (or 2 and 3) of d as f32 (exact).
template <bool HI>
__device__ __forceinline__ v2f e4m3_pair(uint32_t d) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, 1.0f, HI);
}

// e2m1 codes of byte B of d (low nibble first) as f32 (exact).
template <int B>
__device__ __forceinline__ v2f e2m1_pair(uint32_t d) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, B);
}

// Eight e2m1 codes (a dword) times the block scale s, as four dwords of two
// bf16 patterns each (lower column in the low half).
__device__ __forceinline__ void fp4x8_bf16(uint32_t d, float s, uint32_t* o) {
    const v2f f[4] = {e2m1_pair<0>(d), e2m1_pair<1>(d), e2m1_pair<2>(d), e2m1_pair<3>(d)};
#pragma unroll
    for (int b = 0; b < 4; ++b) o[b] = (as_u32(f[b].x * s) >> 16) | (as_u32(f[b].y * s) & 0xFFFF0000u);
}

// The bf16 slab: one 16-byte chunk (32 codes, one MXFP4 block or two NVFP4
// blocks) per thread per pass. Each code is widened to f32 by the hardware
// conversion and multiplied by its block scale in f32: the product is exact
// (at most 2 x 4 significant bits) and, for a checked slab, a bf16 value, so
// its bf16 pattern is the high half of the f32.
template <int FMT>
__global__ __launch_bounds__(256) void k_fp4_dequant(const uint8_t* __restrict__ codes,
                                                     const uint8_t* __restrict__ scales, int64_t rows, int64_t cols,
                                                     uint16_t* __restrict__ out) {
    const int64_t cpr = cols / 32, n = rows * cpr;
    for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < n; g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = g / cpr, q = g - r * cpr;
        const uint4 v = load_stream16(codes + g * 16);
        float s0, s1;
        if constexpr (FMT == kMX) {
            s0 = s1 = e8m0_to_f32(scales[r * cpr + q]);
        } else {
            const uint32_t two = *reinterpret_cast<const uint16_t*>(scales + r * (cols / 16) + 2 * q);
            const v2f s = e4m3_pair<false>(two);
            s0 = s.x;
            s1 = s.y;
        }
        const uint32_t d[4] = {v.x, v.y, v.z, v.w};
        uint32_t o[16];
#pragma unroll
        for (int k = 0; k < 4; ++k) fp4x8_bf16(d[k], k < 2 ? s0 : s1, o + 4 * k);  // codes 0-15: first scale
        uint4* dst = reinterpret_cast<uint4*>(out + r * cols + 32 * q);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        dst[2] = make_uint4(o[8], o[9], o[10], o[11]);
        dst[3] = make_uint4(o[12], o[13], o[14], o[15]);
    }
}

// ---------------------------------------------------------------------------
// The native GEMV.
//
// The products run on gfx950's v_mfma_f32_16x16x32_bf16, which accumulates in
// f32 (its sums are as accurate as f32 additions; the scaled FP8 x FP4
// instruction, by contrast, keeps only about 13 bits below its largest
// product). Both operands are decoded in registers to exact bf16 values:
//   A (16 rows): the activation codes times their power-of-two scale, through
//     the scaled conversion v_cvt_scalef32_pk_bf16_fp8;
//   B (16 columns = 16 weight rows): the e2m1 codes through
//     v_cvt_scalef32_pk_bf16_fp4, with the MXFP4 block scale folded into that
//     conversion (a power of two), or unscaled for NVFP4.
// One instruction takes 32 columns, one MXFP4 block: lane group g (lanes
// 16g .. 16g+15) supplies the block's columns 8g .. 8g+7 to both operands.
//
// MXFP4: A row i is token i (rows past M repeat the last token and are not
// stored); the instruction accumulates every block of every step into the
// tile's f32 accumulator.
// NVFP4: the e4m3 block scale of 16 columns cannot be folded into a bf16
// operand exactly in one conversion, so a row of A is a token restricted to
// one 16-column block of the instruction's 32 columns (zeros elsewhere):
// result element (row, n) is that block's sum for weight row n. Each lane
// multiplies its results by their e4m3 scales in f32 (fused multiply-add)
// into four accumulators per token, added at the end of the unit (the order
// is stated at ex_compute_phase). Panels: A row s of token group o is token
// 8o + s/2, block parity s % 2, one instruction per 32-column chunk. One
// token: the four chunks of a step share one accumulator chain, each chunk
// in rows of its own (ex_nv_one_phase).
//
// A unit is R tiles of 16 weight rows of one linear across all its columns,
// 128 columns (a step) at a time, WIN steps per pipeline window. Units are
// numbered over the list in order; wave w of W takes units w, w + W, ...
// Two register sets hold a wave's consecutive windows; as the matrix work of
// a window consumes each phase (step pair) of its set, that phase is refilled
// with the loads of the window after next, so loads stay in flight while the
// wave computes.
//
// Memory access. Every load reads whole 128-byte lines: a weight load covers
// 8 rows x 128 bytes (two steps of each row; lane l reads row l % 8, bytes
// 16 (l / 8) .. +15), and three exchanges of a lane bit with a register bit
// (permlane32, permlane16, and a row-of-16 rotation by 8 under a bank mask) turn
// the two loads of a tile into the instruction operands of both steps. The
// activation codes of a step are read as one 32-column block per lane group
// and exchanged likewise (permlane32, permlane16). Each lane group loads the
// block scales (and the activation scale) of a different step of the window
// and the exchanges hand every lane those of all the window's steps.
// Kernels with 4-step windows read the weights as 4 rows x 256 bytes per
// load, through LDS (weights_to_lds); the MXFP4 panels among them read the
// activation codes as whole lines too and hand them over through LDS
// (ex_xa). One activation row (template flag ONE, the decode case) reads the
// activation as one 8-byte piece per lane and step pair, handed to the
// token's rows by row shifts. Every variant computes the same bits for a
// token.

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

struct alignas(64) ExLin {
    const uint8_t* w;   // codes [rows, K/2]
    const uint8_t* sc;  // block scales [rows, K/32] (MXFP4) or [rows, K/16] (NVFP4)
    const uint8_t* xq;  // activation codes [M, K]
    const uint8_t* xs;  // activation scale codes [M, K/128]
    float* y;           // [M, rows]
    int64_t rows;
    int32_t K, M;
    float g;            // output scale
    int32_t pad;
};
static_assert(sizeof(ExLin) == kSeqDescBytes, "descriptor size of the plan");

// A-operand groups (NVFP4: 8 tokens each), row tiles per unit and steps per
// window.
constexpr int ex_groups(int fmt, int M) { return fmt == kMX || M <= 8 ? 1 : 2; }
constexpr int ex_tiles(int, int) { return 2; }
constexpr int ex_win(int, int O) { return O == 1 ? 4 : 2; }
// Kernels whose weights go through LDS as 4-row x 256-byte loads (ExXchg):
// those with windows of 4 steps (all but NVFP4 panels of more than 8 rows,
// whose windows are 2 steps).
constexpr bool ex_xl(int, int win, bool) { return win == 4; }
// MXFP4 panels of those kernels read the activation codes as whole 128-byte
// lines (8 lanes per token and step, two loads of 8 tokens) and hand them
// over through LDS too (ExXchg). NVFP4 panels keep their exchanges: the extra
// operand registers would cost them their second wave per SIMD.
constexpr bool ex_xa(int fmt, int win, bool one) { return fmt == kMX && ex_xl(fmt, win, one) && !one; }
// f32 accumulators (v4f) of a wave: one per tile and token group; NVFP4
// panels two (chunks k of even and of odd index, ex_compute_phase).
constexpr int ex_nacc(int fmt, int R, int O, bool one) { return R * O * (fmt == kNV && !one ? 2 : 1); }

// A unit's loads go through buffer resources: a resource in scalar
// registers (base, byte count) plus a 32-bit per-lane offset that is fixed for
// the unit, so a load needs no vector arithmetic. The weight and block-scale
// resources of a phase start at its first step and end at the linear's last
// byte: the hardware's range check returns zeros for any offset past that, so
// a step past a row's end (in a last, partial window) reads the next row's
// bytes, or zeros after the linear's last row, and never leaves the buffers.
// Those steps are dropped in ex_compute_phase.
template <int R, int O, bool ONE, bool WL>
struct ExUnit {
    const uint8_t* w;    // the unit's first row of codes
    const uint8_t* sc;   // its first row of block scales
    const uint8_t* xq;
    const uint8_t* xs;
    int64_t w_left;      // bytes of codes from w to the linear's end
    int64_t sc_left;     // bytes of block scales from sc to the linear's end
    int32_t xq_bytes;    // M * K
    int32_t xs_bytes;    // M * K / 128
    uint32_t woff[R][2]; // windows of 2 steps: lane's row in tile t, load h (rows 8h .. 8h+7) + its chunk
    uint32_t soff[R];    // lane: offset of the block scales of its row n of tile t + its lane group's step
    uint32_t xoff[O];    // lane: its token's codes + its 32-column block (kPastEnd: a row past M)
    uint32_t xsoff[O];   // lane: its token's row of activation scales + its lane group's step (likewise)
    // ONE (a single token): one 8-byte load per step pair. MXFP4: lane
    // (n, g) reads the 8 codes of piece p = n / 2 (step p / 4 of the pair,
    // columns 32 (p % 4) + 8g .. +7); NVFP4: see ex_nv_one_phase. xhi
    // selects the lanes of the pair's second step.
    uint32_t xoff1, xhi;
    // ex_xa kernels: lane l of load i reads token 8i + l / 8, bytes
    // 16 (l % 8) .. +15 of each step (kPastEnd: a token >= M, so that load 1
    // reads nothing below 9 tokens)
    uint32_t xline[ONE || WL ? 0 : 2];
    // ex_xl kernels: weight load (q, t, h) reads rows 16t + 8h + 4q .. +3 of
    // the unit, 256 bytes (the window's 4 steps) each; lane l: row l / 16,
    // bytes 16 (l % 16) .. +15, at offset wq[q][t][h] (rows past the end
    // repeat the last). NVFP4 panels, short of registers, keep one lane base
    // instead and add (16t + 8h + 4q) half per load; their rows past the
    // linear's end read zeros (the range check) and are not stored.
    uint32_t wq[WL ? 0 : 2][R][2];
    uint32_t wlane;
    int32_t half;
};

// WL: the per-load lane base of NVFP4 panels (ExUnit::wlane).
template <int FMT, int R, int O, bool ONE>
using ExUnitT = ExUnit<R, O, ONE, FMT == kNV && !ONE>;

constexpr int kBufferWord3 = 0x00020000;  // buffer resource word 3 on gfx9-family targets: raw 32-bit data
constexpr uint32_t kPastEnd = 0x40000000u;   // a lane offset past every resource's end (all are < 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ex_rsrc(const void* base, int64_t bytes) {
    const int64_t n = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kBufferWord3);
}

template <int FMT, int R, int O, int WIN, bool ONE>
struct ExWin {
    uint4 b[WIN / 2][R][2];                      // weights: step pair, tile, load
    typename std::conditional<FMT == kMX, uint32_t, uint2>::type bs[R];  // block scales of one step of the window
    // activation codes: the lane group's 32-column block of each step
    // [step][o][half]; ONE: the step pair's single 8-byte load [pair][0][0]
    typename std::conditional<ONE, uint2, uint4>::type a[ONE ? WIN / 2 : WIN][O][ONE ? 1 : 2];
    uint32_t as[O];                              // activation scale code of one step of the window
};

// Every byte is a named scalar field (ExLin is 64-byte aligned): copies of a
// position then copy fields only, which the compiler keeps in registers or
// drops; implicit padding was copied through scratch memory.
struct ExPos {
    int64_t u, v;  // unit (list numbering) and unit within its linear
    int32_t win, j;
    int32_t more;  // 0: past the wave's last window (the position repeats the last one)
    int32_t spare0;
    int64_t spare1, spare2, spare3, spare4;
    ExLin d;
};
static_assert(sizeof(ExPos) == 64 + sizeof(ExLin), "no padding in a position");

__device__ __forceinline__ int ex_steps(const ExLin& d) { return d.K / kStepCols; }
template <int WIN>
__device__ __forceinline__ int ex_nwin(const ExLin& d) { return (ex_steps(d) + WIN - 1) / WIN; }

template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_unit(ExUnitT<FMT, R, O, ONE>& U, const ExLin& d, int64_t v, int lane) {
    const int64_t r0 = v * (R * kTileRows);
    const int n = lane & 15, g = lane >> 4, c = lane >> 3;
    const int64_t half = d.K / 2, sper = d.K / (FMT == kMX ? 32 : 16);
    U.w = d.w + r0 * half;
    U.sc = d.sc + r0 * sper;
    U.xq = d.xq;
    U.xs = d.xs;
    U.w_left = (d.rows - r0) * half;
    U.sc_left = (d.rows - r0) * sper;
    const int nb = d.K / kActBlock;
    U.xq_bytes = d.M * d.K;
    U.xs_bytes = d.M * nb;
    const uint32_t chunk = 64 * (c >> 2) + 16 * (c & 3);  // the lane's 16 bytes of a step pair's 128
#pragma unroll
    for (int t = 0; t < R; ++t) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // rows past the end repeat the last
            const int64_t row = min(r0 + t * kTileRows + 8 * h + (lane & 7), d.rows - 1) - r0;
            U.woff[t][h] = (uint32_t)(row * half) + chunk;
        }
        U.soff[t] = (uint32_t)((min(r0 + t * kTileRows + n, d.rows - 1) - r0) * sper) +
                    (FMT == kMX ? 4 : 8) * (g % WIN);
    }
    // A row of the matrix instruction holds a token (NVFP4: 8o + row / 2);
    // rows of tokens >= M are never stored, so their lanes read nothing: an
    // offset past the resource's end makes the range check return zeros
    // without touching memory (at M = 1, 15 of every 16 lanes).
#pragma unroll
    for (int o = 0; o < O; ++o) {
        const int tok = FMT == kMX ? n : 8 * o + (n >> 1);
        const bool live = tok < d.M;
        U.xoff[o] = live ? (uint32_t)(tok * d.K + 32 * g) : kPastEnd;
        U.xsoff[o] = live ? (uint32_t)(tok * nb) + g % WIN : kPastEnd;
    }
    if constexpr (ex_xl(FMT, WIN, ONE)) {
        if constexpr (FMT == kNV && !ONE) {
            U.wlane = (uint32_t)((lane >> 4) * half) + 16 * (lane & 15);
            U.half = (int32_t)half;
        } else {
#pragma unroll
            for (int q = 0; q < 2; ++q)
#pragma unroll
                for (int t = 0; t < R; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int64_t row = min(r0 + 16 * t + 8 * h + 4 * q + (lane >> 4), d.rows - 1) - r0;
                        U.wq[q][t][h] = (uint32_t)(row * half) + 16 * (lane & 15);
                    }
        }
    }
    if constexpr (ex_xa(FMT, WIN, ONE)) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int tok = 8 * i + (lane >> 3);
            U.xline[i] = tok < d.M ? (uint32_t)(tok * d.K + 16 * (lane & 7)) : kPastEnd;
        }
    }
    if constexpr (ONE && FMT == kMX) {
        const int pc = n >> 1;
        U.xoff1 = (uint32_t)(32 * (pc & 3) + 8 * g);
        U.xhi = pc >= 4 ? ~0u : 0u;
    } else if constexpr (ONE) {
        // lane n of groups 0, 1 (n of groups 2, 3 less 8), n < 8: chunk
        // k = (0, 2, 1, 3)[n / 2] of step n % 2 of the pair; the other lanes
        // read nothing
        const bool mine = (g >> 1) == (n >> 3);
        const int i = n & 7, kc = (i >> 1) == 1 ? 2 : (i >> 1) == 2 ? 1 : i >> 1;
        U.xoff1 = mine ? (uint32_t)(32 * kc + 8 * g) : kPastEnd;
        U.xhi = mine && (i & 1) ? ~0u : 0u;
        U.xsoff[0] = (uint32_t)(g % WIN);  // every row of A carries the token
    }
}

template <bool LIST, int WIN>
__device__ __forceinline__ ExPos ex_next(const ExPos& p, const ExLin* lin, const int64_t* pre, int64_t W,
                                         int64_t total) {
    ExPos n = p;
    if (!p.more) return n;
    if (p.win + 1 < ex_nwin<WIN>(p.d)) {
        n.win = p.win + 1;
    } else if (p.u + W < total) {
        n.u = p.u + W;
        n.v = p.v + W;
        n.win = 0;
        if constexpr (LIST) {
            if (n.u >= pre[n.j + 1]) {
                do ++n.j;
                while (n.u >= pre[n.j + 1]);
                n.d = lin[n.j];
                n.v = n.u - pre[n.j];
            }
        }
    } else {
        n.more = 0;
    }
    return n;
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff, bool stream) {
    const auto v = stream ? __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 2)   // nontemporal
                          : __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, soff, 0);
    return make_uint4(v[0], v[1], v[2], v[3]);
}

// The loads of phase q (steps 2q and 2q + 1) of window `win` of a unit; phase 0
// also loads the window's block scales and activation scales. No branch:
// every window issues the same loads. The activation steps are clamped to
// the last step (uniformly); the weight and scale resources of a step past
// the end read what ExUnit describes.
template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_issue_weights(ExWin<FMT, R, O, WIN, ONE>& b, const ExUnitT<FMT, R, O, ONE>& U, int win,
                                                 int q) {
    if constexpr (ex_xl(FMT, WIN, ONE)) {  // 4 rows x 256 bytes per load (see ExXchg)
        const __amdgpu_buffer_rsrc_t wr = ex_rsrc(U.w + 256 * win, U.w_left - 256 * win);
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint32_t off = FMT == kNV && !ONE ? U.wlane + (uint32_t)((16 * t + 8 * h + 4 * q) * U.half)
                                                        : U.wq[q][t][h];
                b.b[q][t][h] = buf_load16(wr, off, 0, true);
            }
    } else {
        const int sp = win * WIN + 2 * q;  // first step of the phase
        const __amdgpu_buffer_rsrc_t wr = ex_rsrc(U.w + 64 * sp, U.w_left - 64 * sp);
#pragma unroll
        for (int t = 0; t < R; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) b.b[q][t][h] = buf_load16(wr, U.woff[t][h], 0, true);
    }
}

// The rest of a phase's loads: block and activation scales (phase 0) and
// activation codes.
template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_issue_rest(ExWin<FMT, R, O, WIN, ONE>& b, const ExUnitT<FMT, R, O, ONE>& U, int steps,
                                              int win, int q) {
    const int s0 = win * WIN;
    const int sp = s0 + 2 * q;  // first step of the phase
    if (q == 0) {
        constexpr int SB = FMT == kMX ? 4 : 8;  // block-scale bytes of a row per step
        const __amdgpu_buffer_rsrc_t sr = ex_rsrc(U.sc + SB * s0, U.sc_left - SB * s0);
#pragma unroll
        for (int t = 0; t < R; ++t) {
            if constexpr (FMT == kMX) {
                b.bs[t] = __builtin_amdgcn_raw_buffer_load_b32(sr, (int)U.soff[t], 0, 0);
            } else {
                const auto v = __builtin_amdgcn_raw_buffer_load_b64(sr, (int)U.soff[t], 0, 0);
                b.bs[t] = make_uint2(v[0], v[1]);
            }
        }
    }
    const __amdgpu_buffer_rsrc_t xr = ex_rsrc(U.xq, U.xq_bytes);
    if constexpr (ONE) {
        // both steps of the pair in one load (a step past the end repeats the last)
        const int j0 = min(sp, steps - 1);
        const uint32_t d1 = (uint32_t)(min(sp + 1, steps - 1) - j0) * kStepCols;  // 0 or one step, uniform
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(xr, (int)(U.xoff1 + (U.xhi & d1)), kStepCols * j0, 0);
        b.a[q][0][0] = make_uint2(v[0], v[1]);
    } else if constexpr (ex_xa(FMT, WIN, ONE)) {
#pragma unroll
        for (int s = 2 * q; s < 2 * q + 2; ++s) {
            const int j = min(s0 + s, steps - 1);
#pragma unroll
            for (int i = 0; i < 2; ++i) b.a[s][0][i] = buf_load16(xr, U.xline[i], kStepCols * j, false);
        }
    } else {
#pragma unroll
        for (int s = 2 * q; s < 2 * q + 2; ++s) {
            const int j = min(s0 + s, steps - 1);
#pragma unroll
            for (int o = 0; o < O; ++o) {
                b.a[s][o][0] = buf_load16(xr, U.xoff[o], kStepCols * j, false);
                b.a[s][o][1] = buf_load16(xr, U.xoff[o] + 16, kStepCols * j, false);
            }
        }
    }
    if (q == 0) {
        const __amdgpu_buffer_rsrc_t ar = ex_rsrc(U.xs + s0, U.xs_bytes - s0);
#pragma unroll
        for (int o = 0; o < O; ++o) b.as[o] = __builtin_amdgcn_raw_buffer_load_b8(ar, (int)U.xsoff[o], 0, 0);
    }
}

template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_issue_phase(ExWin<FMT, R, O, WIN, ONE>& b, const ExUnitT<FMT, R, O, ONE>& U, int steps,
                                               int win, int q) {
    ex_issue_weights(b, U, win, q);
    ex_issue_rest(b, U, steps, win, q);
}

template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_issue(ExWin<FMT, R, O, WIN, ONE>& b, const ExUnitT<FMT, R, O, ONE>& U, int steps,
                                         int win) {
#pragma unroll
    for (int q = 0; q < WIN / 2; ++q) ex_issue_phase(b, U, steps, win, q);
}

// Exchange of lane bit 5 (permlane32) or 4 (permlane16) with the index of a
// register pair (x, y): afterwards x holds, in the lanes with that bit set,
// y's values from the lanes with it clear, and y the reverse.
__device__ __forceinline__ void swap32(uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
    x = r[0];
    y = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& x, uint32_t& y) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
    x = r[0];
    y = r[1];
}
// The two loads of a tile (L[h][d]: load h, dword d; lane l holds row
// (l % 8) + 8h, chunk l / 8 of the step pair's 128 bytes) -> the operands
// op[s][k] of step s of the pair, 32-column block k: lane (n, g) = (l % 16,
// l / 16) holds row n, columns 8g .. 8g+7 of the block. Chunk bits
// (c2 c1 c0) = lane bits (5 4 3) become (s, k1, k0) = register bits, and
// (d1, d0, h) become lane bits (5, 4, 3).
__device__ __forceinline__ void weights_to_operands(const uint4 (&ld)[2], uint32_t (&op)[2][4]) {
    uint32_t L[2][4] = {{ld[0].x, ld[0].y, ld[0].z, ld[0].w}, {ld[1].x, ld[1].y, ld[1].z, ld[1].w}};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        swap32(L[h][0], L[h][2]);  // d1 <-> lane bit 5
        swap32(L[h][1], L[h][3]);
        swap16(L[h][0], L[h][1]);  // d0 <-> lane bit 4
        swap16(L[h][2], L[h][3]);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) swap_lane_bit3(L[0][d], L[1][d]);  // h <-> lane bit 3
    // register (h, d1, d0) now holds chunk c = 4 d1 + 2 d0 + h: step d1, block 2 d0 + h
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int k = 0; k < 4; ++k) op[s][k] = L[k & 1][2 * s + (k >> 1)];
}

// The 32 activation codes of block g held by lane group g (two 16-byte loads,
// dword pairs p = 0..3 = columns 8p .. 8p+7) -> for each block k the 8 codes
// of columns 8g .. 8g+7 (dword pair k).
__device__ __forceinline__ void act_to_operands(const uint4 (&ld)[2], uint2 (&op)[4]) {
    uint32_t D[8] = {ld[0].x, ld[0].y, ld[0].z, ld[0].w, ld[1].x, ld[1].y, ld[1].z, ld[1].w};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        swap32(D[0 + e], D[4 + e]);  // pair bit 1 <-> lane bit 5
        swap32(D[2 + e], D[6 + e]);
        swap16(D[0 + e], D[2 + e]);  // pair bit 0 <-> lane bit 4
        swap16(D[4 + e], D[6 + e]);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) op[k] = make_uint2(D[2 * k], D[2 * k + 1]);
}

// One value per lane group (the lane group's step of the window) -> the
// values of the first WIN lane groups, in every lane.
template <int WIN>
__device__ __forceinline__ void gather_groups(uint32_t v, uint32_t (&out)[WIN]) {
    uint32_t a = v, b = v;
    if constexpr (WIN == 4) {
        swap32(a, b);  // a: groups 0, 1; b: groups 2, 3 (in both halves)
        uint32_t a1 = a, b1 = b;
        swap16(a, a1);
        swap16(b, b1);
        out[0] = a;
        out[1] = a1;
        out[2] = b;
        out[3] = b1;
    } else {
        swap16(a, b);  // groups 0 and 1 (2 and 3 repeat them)
        out[0] = a;
        out[1] = b;
    }
}

// Eight e2m1 codes -> bf16 operand, times the power-of-two scale s.
__device__ __forceinline__ v8bf fp4x8_operand(uint32_t d, float s) {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 0);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 1);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 2);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, s, 3);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// Eight e4m3 codes -> bf16 operand, times the power-of-two scale s.
__device__ __forceinline__ v8bf fp8x8_operand(uint2 d, float s) {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.x, s, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.x, s, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.y, s, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d.y, s, true);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}


// Every step's block scales and activation scales of a window, from the lane
// groups that loaded them (MXFP4 uses ws only; NVFP4 ws and ws_hi).
template <int R, int O, int WIN>
struct ExScales {
    uint32_t ws[R][WIN], ws_hi[R][WIN], as[O][WIN];
};

template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_gather(const ExWin<FMT, R, O, WIN, ONE>& b, ExScales<R, O, WIN>& S) {
#pragma unroll
    for (int t = 0; t < R; ++t) {
        if constexpr (FMT == kMX) {
            gather_groups<WIN>(b.bs[t], S.ws[t]);
        } else {
            gather_groups<WIN>(b.bs[t].x, S.ws[t]);
            gather_groups<WIN>(b.bs[t].y, S.ws_hi[t]);
        }
    }
#pragma unroll
    for (int o = 0; o < O; ++o) gather_groups<WIN>(b.as[o], S.as[o]);
}

// The matrix work of phase q (steps 2q, 2q + 1) of a window.
// MXFP4: acc[t] holds token rows x weight rows of tile t.
// NVFP4 accumulation order (every kernel, so every panel height gives the
// same bits): each token has four f32 accumulators B(p, j), p the parity of a
// 16-column block within its 32-column chunk k, j = k % 2. Step by step, and
// within a step chunk j, then chunk j + 2, B(p, j) += s * c with c the
// chunk's block sum (one matrix instruction's row) and s its e4m3 scale
// (fused multiply-add). The output is g ((B(0,0) + B(0,1)) + (B(1,0) + B(1,1))).
// Panels: acc[(t O + o) 2 + j] register e holds, for weight row l % 16,
// B(e % 2, j) of token 8o + 2(l/16) + e/2.
// Lane n + M of each row of 16 lanes into lane n (lanes past the row's end
// read 0): the piece loaded by lane 2p reaches lanes 0 and 1 with M = 2p.
template <int M>
__device__ __forceinline__ uint2 row_shift(uint2 v) {
    if constexpr (M == 0) {
        return v;
    } else {
        constexpr int ctrl = 0x100 + M;  // row_shl:M
        return make_uint2((uint32_t)__builtin_amdgcn_mov_dpp((int)v.x, ctrl, 0xF, 0xF, true),
                          (uint32_t)__builtin_amdgcn_mov_dpp((int)v.y, ctrl, 0xF, 0xF, true));
    }
}

// The single-token kernels read the weights of a window (32 rows x 256
// bytes) as 8 loads of 4 rows x 256 bytes: runs of 256 bytes read faster than
// k_expert's pieces of 128 bytes of 8 rows (routed-expert sweep, MXFP4: 81.8
// against 75.9% of HBM peak with the same arithmetic). The loads go to the
// wave's part of LDS as they are and come back in the matrix instruction's
// operand layout (so no lane exchanges either), which frees their registers
// for the window after next before the matrix work starts.
// Region (dwords): block (step s, tile t) at (2s + t) kExBlkDw + 8s, holding
// [row n (stride kExRowDw)][8-column group g][32-column block k]. The row
// padding (20 dwords for 16) puts the 8 lanes of a 16-byte read on distinct
// banks, the 8s shift does the same for the 32 lanes of a write.
constexpr int kExRowDw = 20;
constexpr int kExBlkDw = kTileRows * kExRowDw;
__host__ __device__ constexpr int ex_blk(int s, int t) { return (2 * s + t) * kExBlkDw + 8 * s; }
constexpr int kExXchgDw = ex_blk(3, 1) + kExBlkDw;
static_assert(kExXchgDw * 4 <= kExWaveLdsBytes, "the exchange region fits a wave's LDS part");

// Activation region (ex_xa kernels), after the weights: the two steps of a
// phase, [step][token (row stride kExActRowDw)][128 bytes], 8 tokens per load
// that carries any; the 4-dword row padding spreads a step's 8-byte operand
// reads over the banks.
constexpr int kExActRowDw = 36;
__host__ __device__ constexpr int ex_act_step_dw(int M) { return (M > 8 ? 16 : 8) * kExActRowDw; }
static_assert((kExXchgDw + 2 * ex_act_step_dw(16)) * 4 <= kExWaveLdsBytes, "both regions fit a wave's LDS part");

struct ExXchg {
    uint32_t* lds;  // the workgroup's LDS
    uint32_t w;     // lane l of a load: its 16 bytes (row l / 16, step (l % 16) / 4, block l % 4), in dwords
    uint32_t r;     // lane (n, g): its reads (row n, group g), in dwords
    uint32_t a;     // the activation region
    uint32_t astep; // its step stride, in dwords
    int32_t an;     // loads per step that carry tokens (1 or 2)
};

__device__ __forceinline__ ExXchg ex_xchg(float* lds, int wave, int lane, int M) {
    const uint32_t base = (uint32_t)wave * (kExWaveLdsBytes / 4);
    const int st = (lane & 15) >> 2;
    ExXchg x;
    x.lds = reinterpret_cast<uint32_t*>(lds);
    x.w = base + (uint32_t)(ex_blk(st, 0) + (lane >> 4) * kExRowDw + (lane & 3));
    x.r = base + (uint32_t)((lane & 15) * kExRowDw + 4 * (lane >> 4));
    x.a = base + (uint32_t)kExXchgDw;
    x.astep = (uint32_t)ex_act_step_dw(M);
    x.an = M > 8 ? 2 : 1;
    return x;
}

// The activation lines of phase q (steps 2q, 2q + 1) into the region: lane l
// of load i writes its 16 bytes at token 8i + l / 8, bytes 16 (l % 8) ...
template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void act_to_lds(const ExWin<FMT, R, O, WIN, ONE>& b, const ExXchg& X, int q, int lane) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i >= X.an) break;
            uint32_t* w = X.lds + X.a + s2 * X.astep + (8 * i + (lane >> 3)) * kExActRowDw + 4 * (lane & 7);
            *reinterpret_cast<uint4*>(w) = b.a[2 * q + s2][0][i];
        }
}

// ... and back as the operands of step 2q + s2 for token tok: piece k holds
// its columns 32k + 8g .. +7 (g = l / 16), as act_to_operands makes them.
__device__ __forceinline__ void act_from_lds(const ExXchg& X, int s2, int tok, int lane, uint2 (&op)[4]) {
    const uint32_t* r = X.lds + X.a + s2 * X.astep + tok * kExActRowDw + 2 * (lane >> 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) op[k] = *reinterpret_cast<const uint2*>(r + 8 * k);
}

// Load (q, t, h) of a window (rows 16t + 8h + 4q .. +3) into the region:
// its groups g = 0..3 go 4 dwords apart ...
__device__ __forceinline__ void weights_to_lds(const uint4& ld, const ExXchg& X, int q, int t, int h) {
    uint32_t* w = X.lds + X.w + t * kExBlkDw + (8 * h + 4 * q) * kExRowDw;
    w[0] = ld.x;
    w[4] = ld.y;
    w[8] = ld.z;
    w[12] = ld.w;
}

// ... and back as the operands op[s][k] of steps 2q, 2q + 1 of tile t, as
// weights_to_operands makes them.
__device__ __forceinline__ void weights_from_lds(const ExXchg& X, int q, int t, uint32_t (&op)[2][4]) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
        const uint4 v = *reinterpret_cast<const uint4*>(X.lds + X.r + ex_blk(2 * q + st, t));
        op[st][0] = v.x;
        op[st][1] = v.y;
        op[st][2] = v.z;
        op[st][3] = v.w;
    }
}

// NVFP4, one token: the four matrix instructions of a step (chunks k) go
// into one accumulator chain, each filling its own rows: row
// 8p + 4(k % 2) + k / 2 of A holds the token restricted to block parity p of
// chunk k (lane groups 2p, 2p + 1), every other row is zero. Result element e
// of lane group h is then the block sum of chunk 2e + h % 2, parity h / 2, so
// lane group h multiplies its two elements by their scales into
// B(h / 2, h % 2), chunk h % 2 first (acc[t] element 0). The activation load
// puts chunk k of step s2 in lane i = 2 idx(k) + s2, idx = (0, 2, 1, 3)[k], of
// groups 0, 1 (lane i + 8 of groups 2, 3): a row shift by
// i - (4(k % 2) + k / 2), which is s2 for k = 0, 1 and s2 + 1 for k = 2, 3,
// brings it to chunk k's row in both halves of the lane groups.
template <int R, int O, int WIN>
__device__ __forceinline__ void ex_nv_one_phase(const uint2 a0, const uint32_t (&wop)[R][2][4],
                                                const ExScales<R, O, WIN>& S, int steps, int win, int q, int lane,
                                                v4f* acc) {
    const int n = lane & 15, g = lane >> 4;
    const uint32_t b = (uint32_t)(2 * (g & 1) + (g >> 1));  // block of element 0 (element 1: 4 + b)
    const uint32_t sel = b | ((4u + b) << 8) | 0x0C0C0000u;  // bytes b of ws, then of ws_hi
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
        const int s = 2 * q + s2;
        if (win * WIN + s >= steps) continue;  // past the row's end: adds nothing (wave-uniform)
        uint2 ap[4];
        if (s2 == 0) {
            ap[0] = row_shift<0>(a0);
            ap[2] = row_shift<1>(a0);
        } else {
            ap[0] = row_shift<1>(a0);
            ap[2] = row_shift<2>(a0);
        }
        ap[1] = ap[0];
        ap[3] = ap[2];
        const float sa = e8m0_cvt_scale<0>(S.as[0][s]);
        v8bf A[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const bool row = n == 8 * (g >> 1) + 4 * (k & 1) + (k >> 1);
            A[k] = fp8x8_operand(row ? ap[k] : make_uint2(0, 0), sa);
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            v4f c = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[k], fp4x8_operand(wop[t][s2][k], 1.0f), c, 0, 0, 0);
            const v2f sc = e4m3_pair<false>(__builtin_amdgcn_perm(S.ws_hi[t][s], S.ws[t][s], sel));
            acc[t][0] = __builtin_fmaf(sc.x, c[0], acc[t][0]);
            acc[t][0] = __builtin_fmaf(sc.y, c[1], acc[t][0]);
        }
    }
}

template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_compute_phase(const ExWin<FMT, R, O, WIN, ONE>& b, const ExScales<R, O, WIN>& S,
                                                 int steps, int win, int q, int lane, const ExXchg& X, v4f* acc) {
    const int g = lane >> 4;
    uint32_t wop[R][2][4];
#pragma unroll
    for (int t = 0; t < R; ++t) {
        if constexpr (ex_xl(FMT, WIN, ONE))
            weights_from_lds(X, q, t, wop[t]);  // stored by ex_stage
        else
            weights_to_operands(b.b[q][t], wop[t]);
    }
    if constexpr (FMT == kNV && ONE) {
        ex_nv_one_phase<R, O, WIN>(b.a[q][0][0], wop, S, steps, win, q, lane, acc);
    } else {
        if constexpr (ex_xa(FMT, WIN, ONE)) act_to_lds(b, X, q, lane);
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int s = 2 * q + s2;
            const bool live = win * WIN + s < steps;  // wave-uniform
            // MXFP4: a step past the row's end (in a last, partial window) adds
            // nothing; a wave-uniform branch skips it.
            if (FMT == kMX && !live) continue;
            v8bf A[4][O];
#pragma unroll
            for (int o = 0; o < O; ++o) {
                uint2 ap[4];
                if constexpr (ONE) {
                    // the token's row n = 0 takes piece 4 s2 + k from lane 2(4 s2 + k)
                    const uint2 a0 = b.a[q][0][0];
                    if (s2 == 0) {
                        ap[0] = row_shift<0>(a0);
                        ap[1] = row_shift<2>(a0);
                        ap[2] = row_shift<4>(a0);
                        ap[3] = row_shift<6>(a0);
                    } else {
                        ap[0] = row_shift<8>(a0);
                        ap[1] = row_shift<10>(a0);
                        ap[2] = row_shift<12>(a0);
                        ap[3] = row_shift<14>(a0);
                    }
                } else if constexpr (ex_xa(FMT, WIN, ONE)) {
                    act_from_lds(X, s2, lane & 15, lane, ap);
                } else {
                    act_to_operands(b.a[s][o], ap);
                }
                const float sa = e8m0_cvt_scale<0>(S.as[o][s]);
                if constexpr (FMT == kMX) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) A[k][o] = fp8x8_operand(ap[k], sa);
                } else {
                    // selector row s_ = lane % 16 keeps 16-column block s_ % 2 of
                    // each instruction, held by lane groups 2(s_ % 2) and 2(s_ % 2) + 1
                    const bool keep = live && (g >> 1) == (lane & 1);
#pragma unroll
                    for (int k = 0; k < 4; ++k) A[k][o] = fp8x8_operand(keep ? ap[k] : make_uint2(0, 0), sa);
                }
            }
#pragma unroll
            for (int t = 0; t < R; ++t) {
                if constexpr (FMT == kMX) {
                    const uint32_t ws = S.ws[t][s];
                    const float sw[4] = {e8m0_cvt_scale<0>(ws), e8m0_cvt_scale<1>(ws), e8m0_cvt_scale<2>(ws),
                                         e8m0_cvt_scale<3>(ws)};
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            A[k][0], fp4x8_operand(wop[t][s2][k], sw[k]), acc[t], 0, 0, 0);
                } else {
                    // e4m3 scales of the step's 8 blocks of 16 columns: block 2k + parity
                    const v2f sc[4] = {e4m3_pair<false>(S.ws[t][s]), e4m3_pair<true>(S.ws[t][s]),
                                       e4m3_pair<false>(S.ws_hi[t][s]), e4m3_pair<true>(S.ws_hi[t][s])};
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const v8bf B = fp4x8_operand(wop[t][s2][k], 1.0f);
#pragma unroll
                        for (int o = 0; o < O; ++o) {
                            const v4f c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                A[k][o], B, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                            v4f& a = acc[(t * O + o) * 2 + (k & 1)];
                            a[0] = __builtin_fmaf(sc[k].x, c[0], a[0]);
                            a[1] = __builtin_fmaf(sc[k].y, c[1], a[1]);
                            a[2] = __builtin_fmaf(sc[k].x, c[2], a[2]);
                            a[3] = __builtin_fmaf(sc[k].y, c[3], a[3]);
                        }
                    }
                }
            }
        }
    }
}

// The unit's outputs y = g * accumulator, handed one by one to put(token,
// row within the unit, value). MXFP4: lane (n, g) holds tokens 4g .. 4g+3 of
// weight row n. NVFP4 (the order of ex_compute_phase): panels, lane (n, g)
// holds tokens 8o + 2g and 8o + 2g + 1, each as four accumulators; one
// token, lane group h holds B(h / 2, h % 2) and the groups are added across
// lanes (every lane ends with the same sum).
template <int FMT, int R, int O, bool ONE, typename Put>
__device__ __forceinline__ void ex_outputs(const ExLin& d, int lane, const v4f* acc, Put put) {
    const int n = lane & 15, g = lane >> 4;
#pragma unroll
    for (int t = 0; t < R; ++t) {
        const int r = t * kTileRows + n;
        if constexpr (FMT == kMX) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tok = 4 * g + e;
                if (tok < d.M) put(tok, r, d.g * acc[t][e]);
            }
        } else if constexpr (ONE) {
            float v = acc[t][0];
            v += __shfl_xor(v, 16);  // B(p, 0) + B(p, 1)
            v += __shfl_xor(v, 32);
            if (g == 0) put(0, r, d.g * v);
        } else {
#pragma unroll
            for (int o = 0; o < O; ++o) {
                const v4f& a0 = acc[(t * O + o) * 2];
                const v4f& a1 = acc[(t * O + o) * 2 + 1];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int tok = 8 * o + 2 * g + j;
                    const float v = (a0[2 * j] + a1[2 * j]) + (a0[2 * j + 1] + a1[2 * j + 1]);
                    if (tok < d.M) put(tok, r, d.g * v);
                }
            }
        }
    }
}

template <int FMT, int R, int O, bool ONE>
__device__ __forceinline__ void ex_store(const ExLin& d, int64_t v, int lane, const v4f* acc) {
    const int64_t r0 = v * (R * kTileRows);
    ex_outputs<FMT, R, O, ONE>(d, lane, acc, [&](int tok, int r, float val) {
        if (r0 + r < d.rows) store_global_f32(d.y + (int64_t)tok * d.rows + r0 + r, val);
    });
}

// Where a finished unit's outputs go. A stream of reads runs markedly slower
// while writes are mixed into it than when the same bytes are written in one
// burst after it (measured with a bare 3 GiB read by 2048 waves: 1 KB written
// per 64 KB read costs 13% of the read rate, the same bytes written at each
// wave's end 6%). From 8 activation rows on, the outputs are 1/50 of the
// bytes a step reads, so each wave keeps the outputs of its first units in its
// own part of the workgroup's LDS and writes them after its last unit; the
// units past what that part holds are written when they finish. Only where
// and when the outputs are stored changes, never their values.
//
// A slot holds one unit's outputs as y holds them: [token][row of the unit],
// M x 32 floats. Where held unit k goes is recorded in lane k of five
// registers (its y address, y's row stride, and its row count with the flag
// for 16-byte stores), so the final writes load nothing but LDS.
constexpr int kExLdsBytes = 80 * 1024;                      // per workgroup: at most 2 per compute unit
constexpr int kExWaveLds = kExLdsBytes / kSeqWaves;         // per wave
static_assert(kExWaveLds == kExWaveLdsBytes, "LDS part of a wave");
constexpr int kExHoldMinM = 8;                              // smallest panel whose outputs are held back
constexpr int kExUnitRows = ex_tiles(kMX, 1) * kTileRows;   // rows of a unit (both formats)
static_assert(ex_tiles(kNV, 2) * kTileRows == kExUnitRows, "one unit height");
static_assert(kMfSeqBlocksPerCU * kExLdsBytes <= 160 * 1024 && (kMfSeqBlocksPerCU + 1) * kExLdsBytes > 160 * 1024,
              "the LDS of a workgroup caps a compute unit at kMfSeqBlocksPerCU of them");

struct ExOut {
    float* lds;      // the wave's part of the workgroup's LDS
    int slots;       // units it holds (0 below kExHoldMinM activation rows)
    int k;           // units finished so far
    uint32_t y_lo, y_hi, rows_lo, rows_hi, left_vec;  // lane k: record of held unit k
};

template <int FMT, int R, int O, bool ONE>
__device__ __forceinline__ void ex_retire(const ExLin& d, int64_t v, int lane, const v4f* acc, ExOut& o) {
    if (o.k < o.slots) {
        const int64_t r0 = v * (R * kTileRows);
        const uint64_t yu = reinterpret_cast<uint64_t>(d.y + r0);
        const bool vec = (d.rows & 3) == 0 && (reinterpret_cast<uint64_t>(d.y) & 15) == 0;
        const uint32_t lv = (uint32_t)min(d.rows - r0, (int64_t)kExUnitRows) | (vec ? 0x10000u : 0u);
        const bool mine = lane == o.k;  // lane k keeps unit k's record
        o.y_lo = mine ? (uint32_t)yu : o.y_lo;
        o.y_hi = mine ? (uint32_t)(yu >> 32) : o.y_hi;
        o.rows_lo = mine ? (uint32_t)d.rows : o.rows_lo;
        o.rows_hi = mine ? (uint32_t)((uint64_t)d.rows >> 32) : o.rows_hi;
        o.left_vec = mine ? lv : o.left_vec;
        float* slot = o.lds + o.k * d.M * kExUnitRows;
        ex_outputs<FMT, R, O, ONE>(d, lane, acc,
                                   [&](int tok, int r, float val) { slot[tok * kExUnitRows + r] = val; });
    } else {
        ex_store<FMT, R, O, ONE>(d, v, lane, acc);
    }
    ++o.k;
}

// After the wave's last unit: the held units go out in order, each as M rows
// of 32 outputs, four per lane (one 16-byte store where the linear allows it).
// (Called from inside the pipeline loop, at the last unit, as in the
// matrix-core sequence: code after the loop makes the compiler keep more
// registers live across it.)
__device__ __forceinline__ void ex_flush(int lane, int M, const ExOut& o) {
    const int held = min(o.k, o.slots);
    constexpr int Q = kExUnitRows / 4;  // lanes per token row
#pragma unroll 1
    for (int k = 0; k < held; ++k) {
        const uint64_t yu =
            ((uint64_t)__builtin_amdgcn_readlane(o.y_hi, k) << 32) | (uint32_t)__builtin_amdgcn_readlane(o.y_lo, k);
        const int64_t rows = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(o.rows_hi, k) << 32) |
                                       (uint32_t)__builtin_amdgcn_readlane(o.rows_lo, k));
        const uint32_t lv = __builtin_amdgcn_readlane(o.left_vec, k);
        const int left = (int)(lv & 0xffffu);
        const bool vec = (lv >> 16) != 0;
        const float* slot = o.lds + k * M * kExUnitRows;
        float* y = reinterpret_cast<float*>(yu);
        for (int i = lane; i < M * Q; i += kLanes) {
            const int tok = i / Q, r = 4 * (i % Q);
            const v4f val = *reinterpret_cast<const v4f*>(slot + tok * kExUnitRows + r);
            float* dst = y + (int64_t)tok * rows + r;
            if (vec && r + 3 < left) {
                typedef __attribute__((address_space(1))) v4f global_v4f;
                __builtin_nontemporal_store(val, (global_v4f*)dst);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (r + e < left) store_global_f32(dst + e, val[e]);
            }
        }
    }
}

// One window of the pipeline on register set `set`: the matrix work of
// window `cur`, phase by phase, each phase's registers refilled with the
// loads of window `nxt` (two windows ahead) as soon as they are consumed, so
// that about two windows of loads stay in flight while the wave computes;
// then, at the end of cur's unit, its outputs; after the wave's last window
// (`last`), what LDS holds. `un` addresses the windows of `set`.
template <int FMT, int R, int O, int WIN, bool ONE>
__device__ __forceinline__ void ex_stage(const ExPos& cur, const ExPos& nxt, bool last, ExUnitT<FMT, R, O, ONE>& un,
                                         ExWin<FMT, R, O, WIN, ONE>& set, int lane, const ExXchg& X, v4f* acc,
                                         ExOut& out) {
    constexpr int NACC = ex_nacc(FMT, R, O, ONE);
    ExScales<R, O, WIN> S;
    ex_gather(set, S);
    if (nxt.win == 0 && nxt.more) ex_unit<FMT, R, O, WIN, ONE>(un, nxt.d, nxt.v, lane);
    const int csteps = ex_steps(cur.d), nsteps = ex_steps(nxt.d);
    if constexpr (ex_xl(FMT, WIN, ONE)) {
        // every load of the window carries all its steps: the whole window
        // goes to LDS, its registers take the weights of window nxt, then the
        // matrix work, then the rest of nxt's loads
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < WIN / 2; ++q)
#pragma unroll
            for (int t = 0; t < R; ++t)
#pragma unroll
                for (int h = 0; h < 2; ++h) weights_to_lds(set.b[q][t][h], X, q, t, h);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < WIN / 2; ++q) ex_issue_weights(set, un, nxt.win, q);
#pragma unroll
        for (int q = 0; q < WIN / 2; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            ex_compute_phase(set, S, csteps, cur.win, q, lane, X, acc);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 0; q < WIN / 2; ++q) ex_issue_rest(set, un, nsteps, nxt.win, q);
    } else {
#pragma unroll
        for (int q = 0; q < WIN / 2; ++q) {
            __builtin_amdgcn_sched_barrier(0);
            ex_compute_phase(set, S, csteps, cur.win, q, lane, X, acc);
            __builtin_amdgcn_sched_barrier(0);  // the phase's registers are free: refill them
            ex_issue_phase(set, un, nsteps, nxt.win, q);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (cur.win + 1 == ex_nwin<WIN>(cur.d)) {
        ex_retire<FMT, R, O, ONE>(cur.d, cur.v, lane, acc, out);
#pragma unroll
        for (int k = 0; k < NACC; ++k) acc[k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        if (last) ex_flush(lane, cur.d.M, out);
    }
}

// LIST: descriptors from the plan (lin, pre); else the one linear `one`.
// Two register sets: set a holds windows p0, p2, ..., set b windows p1, p3, ...
// (consecutive windows of the wave, possibly of different units).
template <int FMT, int R, int O, int WIN, bool LIST, bool ONE>
__global__ __launch_bounds__(kSeqWaves * kLanes) void k_expert(const ExLin* __restrict__ lin,
                                                                const int64_t* __restrict__ pre, int64_t total,
                                                                ExLin one) {
    constexpr int NACC = ex_nacc(FMT, R, O, ONE);
    using Win = ExWin<FMT, R, O, WIN, ONE>;
    using Unit = ExUnitT<FMT, R, O, ONE>;
    extern __shared__ __attribute__((aligned(16))) float ex_lds[];
    const int lane = threadIdx.x % kLanes;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int64_t W = (int64_t)gridDim.x * kSeqWaves;
    ExPos p0;
    p0.u = (int64_t)xcd_contiguous_block() * kSeqWaves + wave;
    if (p0.u >= total) return;
    p0.win = 0;
    p0.j = 0;
    p0.spare0 = 0;
    p0.spare1 = p0.spare2 = p0.spare3 = p0.spare4 = 0;
    p0.more = 1;
    if constexpr (LIST) {
        while (p0.u >= pre[p0.j + 1]) ++p0.j;
        p0.d = lin[p0.j];
        p0.v = p0.u - pre[p0.j];
    } else {
        p0.d = one;
        p0.v = p0.u;
    }
    // Every linear of a list has the same M (the plan checks it).
    const ExXchg X = ex_xchg(ex_lds, wave, lane, p0.d.M);
    ExOut out;
    // the weight exchange (and the activation region) take the start of the wave's part
    const int xchg = (ex_xl(FMT, WIN, ONE) ? kExXchgDw : 0) + (ex_xa(FMT, WIN, ONE) ? 2 * (int)X.astep : 0);
    out.lds = ex_lds + wave * (kExWaveLds / 4) + xchg;
    const int slot_floats = p0.d.M * kExUnitRows;
    out.slots = p0.d.M >= kExHoldMinM ? min(kLanes, (kExWaveLds / 4 - xchg) / slot_floats) : 0;
    out.k = 0;
    out.y_lo = out.y_hi = out.rows_lo = out.rows_hi = out.left_vec = 0;
    Unit ua, ub;
    ex_unit<FMT, R, O, WIN, ONE>(ua, p0.d, p0.v, lane);
    v4f acc[NACC];
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    Win a, b;
    ex_issue(a, ua, ex_steps(p0.d), p0.win);
    ExPos p1 = ex_next<LIST, WIN>(p0, lin, pre, W, total);
    ub = ua;
    if (p1.win == 0 && p1.more) ex_unit<FMT, R, O, WIN, ONE>(ub, p1.d, p1.v, lane);
    ex_issue(b, ub, ex_steps(p1.d), p1.win);
    for (;;) {
        // the window issued into a set follows the one in the other set: it
        // continues that window's unit unless it starts a new one
        const ExPos p2 = ex_next<LIST, WIN>(p1, lin, pre, W, total);
        ua = ub;
        ex_stage(p0, p2, !p1.more, ua, a, lane, X, acc, out);
        if (!p1.more) break;
        const ExPos p3 = ex_next<LIST, WIN>(p2, lin, pre, W, total);
        ub = ua;
        ex_stage(p1, p3, !p2.more, ub, b, lane, X, acc, out);
        if (!p2.more) break;
        p0 = p2;
        p1 = p3;
    }
}

// ---------------------------------------------------------------------------
// Host side

int64_t ex_units(int fmt, int64_t rows, int64_t M) {
    return ceil_div(rows, (int64_t)ex_tiles(fmt, ex_groups(fmt, (int)M)) * kTileRows);
}

int ex_grid(int64_t units) {
    const int cus = device_cus();
    if (cus < 1) return -1;
    const int64_t cap = (int64_t)cus * kMfSeqBlocksPerCU;
    const int64_t need = ceil_div(units, kSeqWaves);
    return (int)(need < cap ? need : cap);
}

template <int FMT, int O, bool LIST, bool ONE>
void ex_launch_o(const ExLin* lin, const int64_t* pre, int64_t total, const ExLin& one, int grid, hipStream_t s) {
    constexpr int R = ex_tiles(FMT, O), WIN = ex_win(FMT, O);
    constexpr int lds = kExLdsBytes;
    k_expert<FMT, R, O, WIN, LIST, ONE><<<dim3((unsigned)grid), dim3(kSeqWaves * kLanes), lds, s>>>(lin, pre, total,
                                                                                                   one);
}

// A single activation row (M = 1) takes the kernels whose activation loads
// serve both steps of a pair at once (ExUnit, ONE).
template <bool LIST>
int ex_launch(int fmt, int M, const ExLin* lin, const int64_t* pre, int64_t total, const ExLin& one, int grid,
              hipStream_t s) {
    (void)hipGetLastError();
    if (fmt == kMX) {
        if (M == 1)
            ex_launch_o<kMX, 1, LIST, true>(lin, pre, total, one, grid, s);
        else
            ex_launch_o<kMX, 1, LIST, false>(lin, pre, total, one, grid, s);
    } else if (ex_groups(kNV, M) == 1) {
        if (M == 1)
            ex_launch_o<kNV, 1, LIST, true>(lin, pre, total, one, grid, s);
        else
            ex_launch_o<kNV, 1, LIST, false>(lin, pre, total, one, grid, s);
    } else {
        ex_launch_o<kNV, 2, LIST, false>(lin, pre, total, one, grid, s);
    }
    return launch_status();
}

bool fmt_ok(int fmt) { return fmt == kMX || fmt == kNV; }

// rows >= 1, cols a multiple of `mult` in [mult, FP8BLK_MAX_COLS], rows * cols bounded.
bool fp4_shape_ok(int64_t rows, int64_t cols, int64_t mult) {
    if (rows < 1 || cols < mult || cols > FP8BLK_MAX_COLS || cols % mult != 0) return false;
    return rows <= (INT64_C(1) << 46) / cols;
}

int ex_check(int fmt, const uint8_t* codes, const uint8_t* scales, float g, int64_t rows, int64_t cols,
             const uint8_t* xq, const uint8_t* xs, int64_t M, const float* y) {
    if (!fmt_ok(fmt) || !codes || !scales || !xq || !xs || !y || !fp4_shape_ok(rows, cols, kStepCols) || M < 1 ||
        M > FP8BLK_MAX_M || !(g - g == 0.0f) || !aligned(codes, 16) || !aligned(xq, 16) || !aligned(y, 4) ||
        !aligned(scales, fmt == kMX ? 4 : 8))
        return FP8BLK_ERR_ARG;
    return FP8BLK_OK;
}

ExLin ex_desc(const uint8_t* codes, const uint8_t* scales, float g, int64_t rows, int64_t cols, const uint8_t* xq,
              const uint8_t* xs, int64_t M, float* y) {
    ExLin d;
    d.w = codes;
    d.sc = scales;
    d.xq = xq;
    d.xs = xs;
    d.y = y;
    d.rows = rows;
    d.K = (int32_t)cols;
    d.M = (int32_t)M;
    d.g = g;
    d.pad = 0;
    return d;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" int fp8blk_act_quant(const uint16_t* x_bf16, int64_t M, int64_t cols, uint8_t* xq, uint8_t* xs,
                                fp8blk_stream_t stream) {
    if (!x_bf16 || !xq || !xs || M < 1 || M > FP8BLK_MAX_M || !shape_ok(1, cols) || !aligned(x_bf16, 16) ||
        !aligned(xq, 16))
        return FP8BLK_ERR_ARG;
    const int nb = (int)ceil_div(cols, kActBlock);
    (void)hipGetLastError();
    k_act_quant<<<dim3((unsigned)nb, (unsigned)M), dim3(kLanes), 0, reinterpret_cast<hipStream_t>(stream)>>>(
        x_bf16, cols, nb, xq, xs);
    return launch_status();
}

extern "C" int fp4_load_check(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                              void* ws, size_t ws_bytes, int64_t* first_bad, fp8blk_stream_t stream) {
    if (first_bad) *first_bad = -1;
    if (!fmt_ok(fmt) || !codes || !scales || !fp4_shape_ok(rows, cols, 32) || !aligned(codes, 16))
        return FP8BLK_ERR_ARG;
    if (!ws || ws_bytes < fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK, rows, cols, 1) || !aligned(ws, 8))
        return FP8BLK_ERR_WORKSPACE;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    auto* verdict = static_cast<unsigned long long*>(ws);
    const int64_t nsc = rows * (cols / fp4_block(fmt));
    int64_t blocks = ceil_div(nsc, 256);
    if (blocks > 4096) blocks = 4096;
    (void)hipGetLastError();
    k_fp4_verdict_init<<<1, 64, 0, s>>>(verdict);
    if (fmt == kMX)
        k_fp4_check<kMX><<<(unsigned)blocks, 256, 0, s>>>(codes, scales, rows, cols, verdict);
    else
        k_fp4_check<kNV><<<(unsigned)blocks, 256, 0, s>>>(codes, scales, rows, cols, verdict);
    if (launch_status() != FP8BLK_OK) return FP8BLK_ERR_HIP;
    unsigned long long host[3] = {kNone, kNone, kNone};
    if (hipMemcpyAsync(host, verdict, sizeof host, hipMemcpyDeviceToHost, s) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return FP8BLK_ERR_HIP;
    const int kinds[3] = {FP8BLK_ERR_SCALE_FF, FP8BLK_ERR_BAD_SCALE, FP8BLK_ERR_INEXACT};
    for (int k = 0; k < 3; ++k)
        if (host[k] != kNone) {
            if (first_bad) *first_bad = (int64_t)host[k];
            return kinds[k];
        }
    return FP8BLK_OK;
}

extern "C" int fp4_dequant_bf16(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                                uint16_t* out_bf16, fp8blk_stream_t stream) {
    if (!fmt_ok(fmt) || !codes || !scales || !out_bf16 || !fp4_shape_ok(rows, cols, 32) || !aligned(codes, 16) ||
        !aligned(out_bf16, 16) || (fmt == kNV && !aligned(scales, 2)))
        return FP8BLK_ERR_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    int64_t blocks = ceil_div(rows * (cols / 32), 256);
    if (blocks > 8192) blocks = 8192;
    (void)hipGetLastError();
    if (fmt == kMX)
        k_fp4_dequant<kMX><<<(unsigned)blocks, 256, 0, s>>>(codes, scales, rows, cols, out_bf16);
    else
        k_fp4_dequant<kNV><<<(unsigned)blocks, 256, 0, s>>>(codes, scales, rows, cols, out_bf16);
    return launch_status();
}

extern "C" int fp4_expert_gemv(int fmt, const uint8_t* codes, const uint8_t* scales, float global_scale,
                               int64_t rows, int64_t cols, const uint8_t* xq, const uint8_t* xs, int64_t M, float* y,
                               fp8blk_stream_t stream) {
    const int st = ex_check(fmt, codes, scales, global_scale, rows, cols, xq, xs, M, y);
    if (st != FP8BLK_OK) return st;
    const int64_t units = ex_units(fmt, rows, M);
    const int grid = ex_grid(units);
    if (grid < 1) return FP8BLK_ERR_HIP;
    const ExLin one = ex_desc(codes, scales, global_scale, rows, cols, xq, xs, M, y);
    return ex_launch<false>(fmt, (int)M, nullptr, nullptr, units, one, grid, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp4_expert_sequence_init(fp8blk_sequence* seq, int fmt, const fp4_expert_linear* linears, int n,
                                        void* ws, size_t ws_bytes, fp8blk_stream_t stream) {
    if (!seq || !fmt_ok(fmt) || !linears || n < 1 || n > FP8BLK_MAX_SEQ) return FP8BLK_ERR_ARG;
    const int64_t M = linears[0].M;
    for (int j = 0; j < n; ++j) {
        const fp4_expert_linear& l = linears[j];
        if (l.M != M ||
            ex_check(fmt, l.codes, l.scales, l.global_scale, l.rows, l.cols, l.xq, l.xs, l.M, l.y) != FP8BLK_OK)
            return FP8BLK_ERR_ARG;
    }
    const size_t bytes = plan_bytes(n);
    if (!ws || ws_bytes < bytes || !aligned(ws, 64)) return FP8BLK_ERR_WORKSPACE;
    std::vector<unsigned char> host(bytes, 0);
    ExLin* d = reinterpret_cast<ExLin*>(host.data());
    int64_t* pre = reinterpret_cast<int64_t*>(host.data() + (size_t)n * sizeof(ExLin));
    pre[0] = 0;
    for (int j = 0; j < n; ++j) {
        const fp4_expert_linear& l = linears[j];
        d[j] = ex_desc(l.codes, l.scales, l.global_scale, l.rows, l.cols, l.xq, l.xs, l.M, l.y);
        pre[j + 1] = pre[j] + ex_units(fmt, l.rows, l.M);
    }
    const int grid = ex_grid(pre[n]);
    if (grid < 1) return FP8BLK_ERR_HIP;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(ws, host.data(), bytes, hipMemcpyHostToDevice, s) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return FP8BLK_ERR_HIP;
    seq->plan = ws;
    seq->units_dense = pre[n];
    seq->units_general = 0;
    seq->n = n;
    seq->arm = fmt == kMX ? FP8BLK_ARM_MXFP4 : FP8BLK_ARM_NVFP4;
    seq->grid_dense = grid;
    seq->grid_general = 0;
    seq->M = (int32_t)M;
    seq->reserved = 0;
    return FP8BLK_OK;
}

extern "C" int fp4_expert_sequence(const fp8blk_sequence* seq, fp8blk_stream_t stream) {
    if (!seq || !seq->plan || (seq->arm != FP8BLK_ARM_MXFP4 && seq->arm != FP8BLK_ARM_NVFP4) || seq->n < 1 ||
        seq->M < 1 || seq->M > FP8BLK_MAX_M || seq->units_dense < 1 || seq->grid_dense < 1)
        return FP8BLK_ERR_ARG;
    const ExLin* lin = static_cast<const ExLin*>(seq->plan);
    const int64_t* pre =
        reinterpret_cast<const int64_t*>(static_cast<const unsigned char*>(seq->plan) + (size_t)seq->n * sizeof(ExLin));
    const int fmt = seq->arm == FP8BLK_ARM_MXFP4 ? kMX : kNV;
    ExLin none{};
    return ex_launch<true>(fmt, seq->M, lin, pre, seq->units_dense, none, seq->grid_dense,
                           reinterpret_cast<hipStream_t>(stream));
}
