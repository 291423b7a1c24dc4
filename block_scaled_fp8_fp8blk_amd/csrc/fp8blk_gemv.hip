// The FP8-blk GEMV and its bf16-slab twin: one kernel template, two weight
// fetchers.
//
// "Module dsv4_gpu" page (memra-engine docs), struct Fp8Dense: the GEMV forms
// e4m3(code) * scale in registers, the same f32 value the bf16 dequant slab
// holds, and keeps the bf16 kernel's accumulation order, so the two arms give
// identical bits. "Struct Dsv4Gpu" page, spec_greedy_batched_with: a batched
// kernel gives the same bits as its single-position twin. Here both follow
// from construction: the two arms instantiate the same template and differ
// only in how a lane obtains its 16 f32 weights, and the summation order of
// an output depends on cols alone.
//
// Reduction order for output (m, r) (the library header states it too):
//   segment t = columns [1024 t, 1024 t + 1024); lane l owns chunk q = 64 t + l;
//   lane partial = FMA chain over the chunk's 16 columns, increasing, from +0.0;
//   segment sum  = pairwise tree over lanes, bit 5 first, ..., bit 0 last;
//   y = P[0] + P[1] + ... + P[T-1], left to right.
//
// Work decomposition (the launch plan; it never changes bits): a workgroup is
// 4 waves. The waves of a workgroup form 4/sw row streams of sw waves each;
// the sw waves of a stream split the segments of its rows (split-K) and meet
// in LDS, where one wave adds the segment sums in order. Each wave handles R
// consecutive rows, so one x chunk feeds R rows.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kLanes;

struct GemvArgs {
    const void* w;       // uint8 codes [rows, K] or uint16 bf16 slab [rows, K]
    const float* grid;   // f32 block scales [ceil(rows/128), GC] (FP8 arm only)
    const uint16_t* x;   // bf16 [M, K]
    float* y;            // f32 [M, rows]
    int64_t rows;
    int K, M, T, GC;
    int sw;              // waves per row stream: 1, 2 or 4
    int tpw;             // segments per wave, ceil(T / sw)
};

enum Kind { kFp8 = 0, kBf16 = 1 };

// Weight fetchers: load the raw bytes of row r, chunk q, then turn them into
// the chunk's 16 f32 weights.
template <int KIND>
struct Fetch;

template <>
struct Fetch<kFp8> {
    struct Raw {
        uint4 c;
        float s;
    };
    __device__ __forceinline__ static Raw load(const GemvArgs& a, int64_t r, int q) {
        const uint8_t* p = static_cast<const uint8_t*>(a.w) + r * a.K + (int64_t)q * kChunk;
        Raw raw;
        raw.c = *reinterpret_cast<const uint4*>(p);
        raw.s = a.grid[(r >> 7) * a.GC + (q >> 3)];  // chunk q lies in column block q / 8
        return raw;
    }
    __device__ __forceinline__ static void weights(const Raw& raw, float* w) { decode16_fp8(raw.c, raw.s, w); }
};

template <>
struct Fetch<kBf16> {
    struct Raw {
        uint4 lo, hi;
    };
    __device__ __forceinline__ static Raw load(const GemvArgs& a, int64_t r, int q) {
        const uint16_t* p = static_cast<const uint16_t*>(a.w) + r * a.K + (int64_t)q * kChunk;
        Raw raw;
        raw.lo = *reinterpret_cast<const uint4*>(p);
        raw.hi = *reinterpret_cast<const uint4*>(p + 8);
        return raw;
    }
    __device__ __forceinline__ static void weights(const Raw& raw, float* w) {
        widen8_bf16(raw.lo, w);
        widen8_bf16(raw.hi, w + 8);
    }
};

template <int KIND, int MT, int R>
__global__ __launch_bounds__(kThreads) void k_gemv(const GemvArgs a) {
    using F = Fetch<KIND>;
    extern __shared__ float part[];  // [row stream][segment][R * MT], used when sw > 1

    const int wave = threadIdx.x / kLanes, lane = threadIdx.x % kLanes;
    const int streams = kWaves / a.sw;
    const int rs = wave / a.sw, sp = wave % a.sw;
    const int64_t r0 = ((int64_t)blockIdx.x * streams + rs) * R;
    const int tb = sp * a.tpw;
    const int te = min(a.T, tb + a.tpw);

    float y[R][MT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) y[i][m] = 0.0f;

    for (int t = tb; t < te; ++t) {
        const int q = t * kLanes + lane;
        const bool active = q * kChunk < a.K;
        float acc[R][MT];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[i][m] = 0.0f;
        if (active) {
            float w[R][kChunk];
#pragma unroll
            for (int i = 0; i < R; ++i) {
                const int64_t r = min(r0 + i, a.rows - 1);
                F::weights(F::load(a, r, q), w[i]);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                if (m < a.M) {
                    const uint16_t* xp = a.x + (int64_t)m * a.K + (int64_t)q * kChunk;
                    float xv[kChunk];
                    widen8_bf16(*reinterpret_cast<const uint4*>(xp), xv);
                    widen8_bf16(*reinterpret_cast<const uint4*>(xp + 8), xv + 8);
#pragma unroll
                    for (int i = 0; i < R; ++i) {
                        float s = 0.0f;
#pragma unroll
                        for (int j = 0; j < kChunk; ++j) s = __builtin_fmaf(w[i][j], xv[j], s);
                        acc[i][m] = s;
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float P = tree64(acc[i][m]);
                if (a.sw == 1) {
                    y[i][m] = (t == 0) ? P : y[i][m] + P;
                } else if (lane == 0) {
                    part[((int64_t)rs * a.T + t) * (R * MT) + i * MT + m] = P;
                }
            }
    }

    if (a.sw > 1) {
        __syncthreads();
        if (sp != 0) return;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float* p = part + (int64_t)rs * a.T * (R * MT) + i * MT + m;
                float v = p[0];
                for (int t = 1; t < a.T; ++t) v = v + p[t * (R * MT)];
                y[i][m] = v;
            }
    }
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m)
                if (r0 + i < a.rows && m < a.M) a.y[(int64_t)m * a.rows + r0 + i] = y[i][m];
    }
}

struct Plan {
    int MT, R, sw;
};

// Plan: a pure function of (rows, cols, M). Enough waves to fill 256 CUs,
// splitting the segments of a row over 2 or 4 waves when rows are few.
Plan make_plan(int64_t rows, int64_t K, int64_t M) {
    Plan p;
    p.MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    p.R = p.MT <= 4 ? 2 : 1;
    const int64_t T = ceil_div(K, kSegCols);
    const int64_t row_waves = ceil_div(rows, p.R);
    p.sw = 1;
    while (p.sw < 4 && p.sw * 2 <= T && row_waves * p.sw < 4096) p.sw *= 2;
    return p;
}

template <int KIND, int MT, int R>
void launch(const GemvArgs& a, hipStream_t s) {
    const int streams = kWaves / a.sw;
    const int64_t blocks = ceil_div(ceil_div(a.rows, R), streams);
    const size_t lds = a.sw > 1 ? (size_t)streams * a.T * R * MT * sizeof(float) : 0;
    k_gemv<KIND, MT, R><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(a);
}

template <int KIND>
int run(const void* w, const float* grid, int64_t rows, int64_t cols, const uint16_t* x, int64_t M, float* y,
        hipStream_t s) {
    const Plan p = make_plan(rows, cols, M);
    GemvArgs a;
    a.w = w;
    a.grid = grid;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.K = (int)cols;
    a.M = (int)M;
    a.T = (int)ceil_div(cols, kSegCols);
    a.GC = (int)ceil_div(cols, kBlock);
    a.sw = p.sw;
    a.tpw = (int)ceil_div(a.T, p.sw);
    if (ceil_div(ceil_div(rows, p.R), kWaves / p.sw) > 0x7fffffff) return FP8BLK_ERR_ARG;
    (void)hipGetLastError();
    switch (p.MT) {
        case 1: launch<KIND, 1, 2>(a, s); break;
        case 2: launch<KIND, 2, 2>(a, s); break;
        case 4: launch<KIND, 4, 2>(a, s); break;
        case 8: launch<KIND, 8, 1>(a, s); break;
        default: launch<KIND, 16, 1>(a, s); break;
    }
    return launch_status();
}

int check_common(const void* w, int64_t rows, int64_t cols, const uint16_t* x, int64_t M, float* y, size_t need,
                 void* ws, size_t ws_bytes) {
    if (!w || !x || !y || !shape_ok(rows, cols) || M < 1 || M > FP8BLK_MAX_M || !aligned(w, 16) ||
        !aligned(x, 16) || !aligned(y, 4))
        return FP8BLK_ERR_ARG;
    if (need > 0 && (!ws || ws_bytes < need)) return FP8BLK_ERR_WORKSPACE;
    return FP8BLK_OK;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" int fp8blk_gemv(const uint8_t* codes, const float* scales_f32, int64_t rows, int64_t cols,
                           const uint16_t* x_bf16, int64_t M, float* y, void* ws, size_t ws_bytes,
                           fp8blk_stream_t stream) {
    const int st = check_common(codes, rows, cols, x_bf16, M, y,
                                fp8blk_workspace_bytes(FP8BLK_OP_GEMV, rows, cols, M), ws, ws_bytes);
    if (st != FP8BLK_OK) return st;
    if (!scales_f32 || !aligned(scales_f32, 4)) return FP8BLK_ERR_ARG;
    return run<kFp8>(codes, scales_f32, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int bf16_gemv_twin(const uint16_t* w_bf16, int64_t rows, int64_t cols, const uint16_t* x_bf16,
                              int64_t M, float* y, void* ws, size_t ws_bytes, fp8blk_stream_t stream) {
    const int st = check_common(w_bf16, rows, cols, x_bf16, M, y,
                                fp8blk_workspace_bytes(FP8BLK_OP_BF16_TWIN, rows, cols, M), ws, ws_bytes);
    if (st != FP8BLK_OK) return st;
    return run<kBf16>(w_bf16, nullptr, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}
