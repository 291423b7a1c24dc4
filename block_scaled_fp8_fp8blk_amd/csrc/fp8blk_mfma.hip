// The matrix-core arm of the FP8-blk GEMV and its bf16-slab twin.
//
// Same operation as fp8blk_gemv ("Module dsv4_gpu" page of memra-engine,
// struct Fp8Dense; "Struct Dsv4Gpu" page, field dense_fp8): weights
// e4m3(code) * block scale times a bf16 activation panel, f32 accumulation.
// Here the products run on gfx950's matrix cores (v_mfma_f32_16x16x32_bf16)
// instead of the vector FMA chains, so the panel stays bound by HBM instead of
// by vector ALU work for every M <= 16.
//
// What is kept from the pages: the weights are decoded in registers to the
// same values the bf16 dequant slab holds (v_cvt_scalef32_pk_bf16_fp8, exact
// for every weight the load check accepts), and the bf16 twin feeds the same
// instruction sequence from the slab, so the two arms of this kernel give
// identical bits ("Module dsv4_gpu", Fp8Dense). A batched call gives the same
// bits as a single-row call ("Struct Dsv4Gpu", spec_greedy_batched_with): the
// activation panel is always padded to 16 rows, and an output never depends
// on another row of the panel.
//
// What differs from fp8blk_gemv: the matrix core sums the 32 products of an
// instruction internally in an order the hardware does not document, so the
// result is not the documented f32 order of fp8blk_gemv and is checked against
// the exact sum by tolerance only.
//
// Order of operations for output (m, r), with T64 = ceil(cols / 64) blocks of
// 64 columns: within block p, lane group kg (0..3) owns columns
// [64 p + 16 kg, 64 p + 16 kg + 16); the first 8 of them form the k-slice of
// one matrix instruction, the last 8 of the next, and both instructions
// accumulate into the same f32 tile. Blocks are visited in increasing order
// inside each of the sw parts the columns are split into (part s covers blocks
// [s * bpp, (s + 1) * bpp)); the sw partial tiles are added in part order.
// The split sw is a function of (rows, cols) only, never of M.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kMfWaves = 4;
constexpr int kMfThreads = kMfWaves * kLanes;
constexpr int kTile = 16;    // rows per matrix tile, and the padded panel
constexpr int kBlk = 64;     // columns per block (two matrix instructions)

struct MfArgs {
    const void* w;        // uint8 codes or uint16 bf16 slab, [rows, K]
    const float* grid;    // f32 block scales (FP8 arm)
    const uint16_t* x;    // bf16 [M, K]
    float* y;             // f32 [M, rows]
    int64_t rows;
    int K, M, GC;
    int nblk;             // ceil(K / 64)
    int sw_log2;          // waves splitting the columns of a tile: 1, 2, 4
    int bpp;              // blocks per part, ceil(nblk / sw)
};

// 16 consecutive weights of one lane as two 8-wide bf16 operands.
template <int KIND>
struct MfFetch;

template <>
struct MfFetch<0> {  // FP8: codes + f32 block scale, decoded in registers
    struct Raw {
        uint4 c;
        float s;
    };
    __device__ __forceinline__ static Raw load(const MfArgs& a, int64_t r, int col) {
        Raw raw;
        raw.c = load_stream16(static_cast<const uint8_t*>(a.w) + r * a.K + col);
        raw.s = a.grid[(r >> 7) * a.GC + (col >> 7)];
        return raw;
    }
    __device__ __forceinline__ static void operands(const Raw& raw, v8bf& lo, v8bf& hi) {
        const uint32_t d[4] = {raw.c.x, raw.c.y, raw.c.z, raw.c.w};
        v2bf p[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            p[2 * k] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], raw.s, false);     // bytes 0, 1
            p[2 * k + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], raw.s, true);  // bytes 2, 3
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            lo[2 * e] = p[e][0];
            lo[2 * e + 1] = p[e][1];
            hi[2 * e] = p[4 + e][0];
            hi[2 * e + 1] = p[4 + e][1];
        }
    }
    __device__ __forceinline__ static Raw zero() { return Raw{make_uint4(0, 0, 0, 0), 1.0f}; }
};

template <>
struct MfFetch<1> {  // bf16 slab
    struct Raw {
        uint4 lo, hi;
    };
    __device__ __forceinline__ static Raw load(const MfArgs& a, int64_t r, int col) {
        const uint16_t* p = static_cast<const uint16_t*>(a.w) + r * a.K + col;
        Raw raw;
        raw.lo = load_stream16(p);
        raw.hi = load_stream16(p + 8);
        return raw;
    }
    __device__ __forceinline__ static void operands(const Raw& raw, v8bf& lo, v8bf& hi) {
        lo = __builtin_bit_cast(v8bf, raw.lo);
        hi = __builtin_bit_cast(v8bf, raw.hi);
    }
    __device__ __forceinline__ static Raw zero() { return Raw{make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)}; }
};

// A wave owns TILES tiles of 16 consecutive rows and one part of the column
// blocks. Lane l = 16 kg + i: matrix row i of each tile, k-group kg, and, for
// the activation operand, panel row m = i (rows m >= M are zero). The blocks
// are taken U at a time: every load of the U blocks (codes, scales, x) is
// issued before the matrix instructions that consume them. Loads are
// unconditional (a block past the part re-reads the part's last block and is
// skipped; a lane past the last column re-reads the last chunk with a zero
// activation operand), so the waits stay per block.
template <int KIND, int TILES, int U>
__global__ __launch_bounds__(kMfThreads) void k_mfma(const MfArgs a) {
    using F = MfFetch<KIND>;
    __shared__ v4f part[kMfWaves][TILES][kLanes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int i = lane % kTile, kg = lane / kTile;
    const int rs = wave >> a.sw_log2, sp = wave & ((1 << a.sw_log2) - 1);
    const int64_t r0 = (((int64_t)blockIdx.x << (2 - a.sw_log2)) + rs) * (TILES * kTile);
    const int pb = sp * a.bpp;
    const int pe = min(a.nblk, pb + a.bpp);
    const bool xrow = i < a.M;
    const int last_col = a.K - 16;
    const uint16_t* xrow_ptr = a.x + (int64_t)min(i, a.M - 1) * a.K;

    v4f acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    for (int p0 = pb; p0 < pe; p0 += U) {
        typename F::Raw raw[U][TILES];
        uint4 xr[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int col = min(min(p0 + u, pe - 1) * kBlk + kg * 16, last_col);
#pragma unroll
            for (int t = 0; t < TILES; ++t) raw[u][t] = F::load(a, min(r0 + t * kTile + i, a.rows - 1), col);
            const uint4* xp = reinterpret_cast<const uint4*>(xrow_ptr + col);
            xr[u][0] = xp[0];
            xr[u][1] = xp[1];
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (p0 + u < pe) {
                const bool live = xrow && (p0 + u) * kBlk + kg * 16 <= last_col;
                const uint4 z = make_uint4(0, 0, 0, 0);
                const v8bf b0 = __builtin_bit_cast(v8bf, live ? xr[u][0] : z);
                const v8bf b1 = __builtin_bit_cast(v8bf, live ? xr[u][1] : z);
#pragma unroll
                for (int t = 0; t < TILES; ++t) {
                    v8bf a0, a1;
                    F::operands(raw[u][t], a0, a1);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc[t], 0, 0, 0);
                    acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc[t], 0, 0, 0);
                }
            }
        }
    }

    if (a.sw_log2 > 0) {
#pragma unroll
        for (int t = 0; t < TILES; ++t) part[wave][t][lane] = acc[t];
        __syncthreads();
        if (sp != 0) return;
        const int nsw = 1 << a.sw_log2;
#pragma unroll
        for (int t = 0; t < TILES; ++t) {
            v4f s = part[wave][t][lane];
            for (int k = 1; k < nsw; ++k) {
                const v4f o = part[wave + k][t][lane];
                s = v4f{s[0] + o[0], s[1] + o[1], s[2] + o[2], s[3] + o[3]};
            }
            acc[t] = s;
        }
    }
    // lane l holds D[4 (l / 16) + e][l % 16]: row 4 kg + e of the tile, panel row i
    if (i < a.M) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t r = r0 + t * kTile + 4 * kg + e;
                if (r < a.rows) a.y[(int64_t)i * a.rows + r] = acc[t][e];
            }
    }
}

// Plan, a function of (rows, cols) only: the columns of a row group are split
// over 2 or 4 waves while fewer than 2048 waves would run; a wave takes TILES
// = 4, 2 or 1 row tiles -- the most that still leaves >= 768 waves, since the
// row tiles of a wave share its activation loads -- and U = 8 / TILES blocks
// per batch of loads. Measured on 12288 x 4096 and 4096 x 4096 at M = 1 and 16.
struct MfPlan {
    int tiles, sw;
};
MfPlan mf_plan(int64_t rows, int64_t K) {
    MfPlan p;
    const int64_t nblk = ceil_div(K, kBlk);
    p.tiles = 4;
    while (p.tiles > 1 && ceil_div(rows, (int64_t)kTile * p.tiles) * 4 < 768) p.tiles /= 2;
    const int64_t groups = ceil_div(rows, (int64_t)kTile * p.tiles);
    p.sw = 1;
    while (p.sw < 4 && p.sw * 2 <= nblk && groups * p.sw < 2048) p.sw *= 2;
    return p;
}

template <int KIND>
int mf_run(const void* w, const float* grid, int64_t rows, int64_t cols, const uint16_t* x, int64_t M, float* y,
           hipStream_t s) {
    const MfPlan p = mf_plan(rows, cols);
    MfArgs a;
    a.w = w;
    a.grid = grid;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.K = (int)cols;
    a.M = (int)M;
    a.GC = (int)ceil_div(cols, kBlock);
    a.nblk = (int)ceil_div(cols, kBlk);
    a.sw_log2 = p.sw == 4 ? 2 : p.sw == 2 ? 1 : 0;
    a.bpp = (int)ceil_div(a.nblk, p.sw);
    const int streams = kMfWaves / p.sw;
    const int64_t blocks = ceil_div(ceil_div(rows, (int64_t)kTile * p.tiles), streams);
    if (blocks > 0x7fffffff) return FP8BLK_ERR_ARG;
    (void)hipGetLastError();
    const dim3 nb((unsigned)blocks), nt(kMfThreads);
    if (p.tiles == 4)
        k_mfma<KIND, 4, 2><<<nb, nt, 0, s>>>(a);
    else if (p.tiles == 2)
        k_mfma<KIND, 2, 4><<<nb, nt, 0, s>>>(a);
    else
        k_mfma<KIND, 1, 8><<<nb, nt, 0, s>>>(a);
    return launch_status();
}

int mf_check(const void* w, int64_t rows, int64_t cols, const uint16_t* x, int64_t M, float* y) {
    if (!w || !x || !y || !shape_ok(rows, cols) || M < 1 || M > FP8BLK_MAX_M || !aligned(w, 16) ||
        !aligned(x, 16) || !aligned(y, 4))
        return FP8BLK_ERR_ARG;
    return FP8BLK_OK;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" int fp8blk_gemv_mfma(const uint8_t* codes, const float* scales_f32, int64_t rows, int64_t cols,
                                const uint16_t* x_bf16, int64_t M, float* y, fp8blk_stream_t stream) {
    const int st = mf_check(codes, rows, cols, x_bf16, M, y);
    if (st != FP8BLK_OK) return st;
    if (!scales_f32 || !aligned(scales_f32, 4)) return FP8BLK_ERR_ARG;
    return mf_run<0>(codes, scales_f32, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int bf16_gemv_twin_mfma(const uint16_t* w_bf16, int64_t rows, int64_t cols, const uint16_t* x_bf16,
                                   int64_t M, float* y, fp8blk_stream_t stream) {
    const int st = mf_check(w_bf16, rows, cols, x_bf16, M, y);
    if (st != FP8BLK_OK) return st;
    return mf_run<1>(w_bf16, nullptr, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}
