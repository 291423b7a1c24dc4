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
// consecutive rows, so one widened x chunk feeds R rows.
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
    const float* xs;     // f32 [K] (scaled-input launches: x = bf16(xc * xs), M = 1)
    float xc;
    uint16_t* xn;        // when set (M = 1): also write bf16(xnc * y) [rows], the next linear's input
    float xnc;
    float* y;            // f32 [M, rows]
    int64_t rows;
    int K, M, T, GC;
    int sw;              // waves per row stream: 1, 2 or 4
    int sw_log2;         // log2(sw)
    int tpw;             // segments per wave, ceil(T / sw)
    int whole;           // 1: cols is a multiple of 1024 (every segment whole; bf16 loads read whole lines)
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
        raw.c = load_stream16(p);
        raw.s = a.grid[(r >> 7) * a.GC + (q >> 3)];  // chunk q lies in column block q / 8
        return raw;
    }
    __device__ __forceinline__ static void weights(const Raw& raw, float* w, bool) {
        decode16_fp8_scaled(raw.c, raw.s, w);
    }
    // Codes only of rows r0 .. r0 + n - 1 (clamped to the last row) of chunk
    // q; the scales are filled in by the caller.
    template <int N, int TPW>
    __device__ __forceinline__ static void load_codes(const GemvArgs& a, int64_t r0, int q, Raw (&raw)[N][TPW], int u) {
        const uint8_t* base = static_cast<const uint8_t*>(a.w) + (int64_t)q * kChunk;
#pragma unroll
        for (int i = 0; i < N; ++i) raw[i][u].c = load_stream16(base + min(r0 + i, a.rows - 1) * a.K);
    }
    // Rows r0 .. r0 + n - 1 (clamped to the last row) of chunk q, into
    // raw[i][u]. n <= 4 rows starting at a multiple of n share one 128-row
    // block, hence one scale load.
    template <int N, int TPW>
    __device__ __forceinline__ static void load_rows(const GemvArgs& a, int64_t r0, int n, int q, Raw (&raw)[N][TPW],
                                                     int u) {
        const uint8_t* base = static_cast<const uint8_t*>(a.w) + (int64_t)q * kChunk;
        const float s = a.grid[(min(r0, a.rows - 1) >> 7) * a.GC + (q >> 3)];
#pragma unroll
        for (int i = 0; i < N; ++i) {
            raw[i][u].c = load_stream16(base + min(r0 + i, a.rows - 1) * a.K);
            raw[i][u].s = s;
        }
    }
};

// The bf16 slab: a chunk is 32 bytes. Loading a lane's own two halves would
// make each load instruction read every other 16 bytes of the segment's 2 KB
// (half of every line it touches). When every segment is whole (a.whole), load
// 0 reads the segment's first KB and load 1 the second, lane m taking 16-byte
// piece 2m (m < 32) or 2(m - 32) + 1, i.e. elements +0 / +512 (m < 32) or
// -504 / +8 (m >= 32) from its own chunk, and swap_lane_halves hands every
// lane its own two halves back before the arithmetic.
template <>
struct Fetch<kBf16> {
    struct Raw {
        uint4 lo, hi;
    };
    __device__ __forceinline__ static Raw load(const GemvArgs& a, int64_t r, int q) {
        const uint16_t* p = static_cast<const uint16_t*>(a.w) + r * a.K + (int64_t)q * kChunk;
        const bool upper = (threadIdx.x & 32) != 0;  // lanes 32..63 of the wave
        const int d0 = a.whole && upper ? -504 : 0, d1 = !a.whole ? 8 : upper ? 8 : 512;
        Raw raw;
        raw.lo = load_stream16(p + d0);
        raw.hi = load_stream16(p + d1);
        return raw;
    }
    __device__ __forceinline__ static void weights(const Raw& raw, float* w, bool whole) {
        uint4 lo = raw.lo, hi = raw.hi;
        if (whole) swap_lane_halves(lo, hi);
        widen8_bf16(lo, w);
        widen8_bf16(hi, w + 8);
    }
    template <int N, int TPW>
    __device__ __forceinline__ static void load_rows(const GemvArgs& a, int64_t r0, int n, int q, Raw (&raw)[N][TPW],
                                                     int u) {
#pragma unroll
        for (int i = 0; i < N; ++i) raw[i][u] = load(a, min(r0 + i, a.rows - 1), q);
    }
    template <int N, int TPW>
    __device__ __forceinline__ static void load_codes(const GemvArgs& a, int64_t r0, int q, Raw (&raw)[N][TPW], int u) {
        load_rows(a, r0, N, q, raw, u);
    }
};

// Row-of-lane layout of a transposed reduction: value j of a group of four
// ends in row kRowOf4[j] of its register; the mapping is its own inverse.
__device__ __forceinline__ int value_in_row(int row) { return row == 1 ? 2 : row == 2 ? 1 : row; }

// Panel kernel: an activation panel of M <= MT rows (also M = 1 when a row has
// more than 16 segments). A wave owns R consecutive rows and walks its
// segments in order, prefetching the next segment's codes while it computes
// the current one. Per segment, each lane decodes its chunk of the R rows
// once, then for every activation row m widens that row's x chunk and runs the
// R fused multiply-add chains; the R * MT lane partials go through the
// transposing reductions (tree64xV). A value keeps the same register and row
// in every segment, so the running sums over segments are plain register adds,
// and the lanes of a row store their own results. With sw > 1 each segment's
// sums go to LDS and the first wave of the row stream adds them in order.
// The fused multiply-add chains of one segment of the panel kernel: for each
// activation row m (rows >= M repeat row M - 1) and weight row i, the lane's
// 16 columns in increasing order from +0.0, into v[i * MT + m]; MASK: +0.0
// where the lane is not live.
template <bool MASK, int MT, int R>
__device__ __forceinline__ void panel_tokens(const GemvArgs& a, const float (&w)[R][kChunk], int qc, bool live,
                                             float* v) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
        const int64_t xrow = min(m, a.M - 1);
        const uint4* xp = reinterpret_cast<const uint4*>(a.x + xrow * a.K + (int64_t)qc * kChunk);
        float xf[kChunk];
        widen8_bf16(xp[0], xf);
        widen8_bf16(xp[1], xf + 8);
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < kChunk; ++j) s = __builtin_fmaf(w[i][j], xf[j], s);
            v[i * MT + m] = MASK && !live ? 0.0f : s;
        }
    }
}

template <int KIND, int MT, int R>
__device__ __forceinline__ void panel_body(const GemvArgs& a, int64_t block) {
    constexpr int V = R * MT;
    constexpr int VP = V < 4 ? 4 : V;
    constexpr int G = VP / 4;
    using F = Fetch<KIND>;
    extern __shared__ float part[];  // [row stream][segment][VP], used when sw > 1

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int rs = wave >> a.sw_log2, sp = wave & ((1 << a.sw_log2) - 1);
    const int64_t r0 = ((block << (2 - a.sw_log2)) + rs) * R;
    const int tb = sp * a.tpw;
    const int te = min(a.T, tb + a.tpw);
    const int last_q = a.K / kChunk - 1;
    const int vrow = value_in_row(lane >> 4);  // value j held by this lane's row

    float y[G];
#pragma unroll
    for (int g = 0; g < G; ++g) y[g] = 0.0f;

    typename F::Raw raw[R][1];
    if (tb < te) F::load_rows(a, r0, R, min(tb * kLanes + lane, last_q), raw, 0);
    for (int t = tb; t < te; ++t) {
        typename F::Raw nxt[R][1];
        if (t + 1 < te) F::load_rows(a, r0, R, min((t + 1) * kLanes + lane, last_q), nxt, 0);
        const int q = t * kLanes + lane;
        const bool live = q <= last_q;
        const int qc = min(q, last_q);
        float w[R][kChunk];
#pragma unroll
        for (int i = 0; i < R; ++i) F::weights(raw[i][0], w[i], a.whole != 0);
        float v[VP];
#pragma unroll
        for (int k = V; k < VP; ++k) v[k] = 0.0f;
        // Every activation row of the tile runs, rows >= M on a copy of row
        // M - 1 (their outputs are never stored), so the x loads carry no
        // branch and the compiler issues them ahead of the arithmetic. Lanes
        // past the last column contribute +0.0; only a ragged last segment
        // has any (wave-uniform test).
        if ((t + 1) * kLanes - 1 <= last_q)
            panel_tokens<false, MT, R>(a, w, qc, true, v);
        else
            panel_tokens<true, MT, R>(a, w, qc, live, v);
        float red[G];
        tree64xV<VP>(v, red);
        if (a.sw_log2 == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) y[g] = (t == 0) ? red[g] : y[g] + red[g];
        } else if ((lane & 15) == 0) {
            float* dst = part + ((int64_t)rs * a.T + t) * VP;
#pragma unroll
            for (int g = 0; g < G; ++g) dst[4 * g + vrow] = red[g];
        }
#pragma unroll
        for (int i = 0; i < R; ++i) raw[i][0] = nxt[i][0];
    }

    if (a.sw_log2 > 0) {
        __syncthreads();
        if (sp != 0) return;
        // lanes 0 .. VP-1: one value each, summed over the segments in order
        if (lane < VP) {
            const float* p = part + (int64_t)rs * a.T * VP + lane;
            float acc = p[0];
            for (int t = 1; t < a.T; ++t) acc = acc + p[(int64_t)t * VP];
            const int i = lane / MT, m = lane % MT;
            if (lane < V && m < a.M && r0 + i < a.rows) a.y[(int64_t)m * a.rows + r0 + i] = acc;
        }
        return;
    }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int vi = 4 * g + vrow;
            const int i = vi / MT, m = vi % MT;
            if (vi < V && m < a.M && r0 + i < a.rows) a.y[(int64_t)m * a.rows + r0 + i] = y[g];
        }
    }
}

// Single-row (M = 1) kernel. A wave owns R consecutive rows x TPW segments
// (R, TPW in {1, 2, 4}): each lane holds R * TPW 16-column chunks in flight,
// the code is straight-line, and every load of the wave (codes, one block
// scale per segment -- R <= 4 consecutive rows from a multiple of R never
// cross a 128-row block --, x) is issued before any arithmetic. The x chunk of
// a segment is widened once and feeds the R rows. The R * TPW lane partials
// then go through transposing 64-lane reductions (tree64xV), which yield
// exactly the per-segment trees of the order above. When a row has more than
// TPW segments they are split over sw = 2 or 4 waves of the workgroup, which
// leave their segment sums in LDS; one wave then adds them in order. Lanes
// whose chunk lies past the last column load a valid chunk and contribute +0.0.
template <int KIND, int R, int TPW, int MT, bool XS = false>
__device__ __forceinline__ void m1_body(const GemvArgs& a, int64_t block) {
    static_assert(!XS || MT == 1, "a scaled input is one activation row");
    constexpr int V = R * TPW * MT;
    constexpr int VP = V < 4 ? 4 : V;  // reductions run in groups of four values
    using F = Fetch<KIND>;
    extern __shared__ float part[];  // [row stream][segment][R][MT], used when sw > 1

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);  // uniform: scalar branches below
    const int lane = threadIdx.x % kLanes;
    const int rs = wave >> a.sw_log2, sp = wave & ((1 << a.sw_log2) - 1);
    const int64_t r0 = ((block << (2 - a.sw_log2)) + rs) * R;
    const int t0 = sp * a.tpw;
    const int nseg = min(a.tpw, a.T - t0);  // wave-uniform; <= 0 for an idle wave
    const int last_q = a.K / kChunk - 1;

    // Loads are unconditional and in the order the arithmetic consumes them,
    // so the compiler can wait for each segment alone (no branch merges the
    // outstanding-load counts). A segment past this wave's range re-reads
    // its last one, a chunk past the last column re-reads the last chunk;
    // both are discarded below. With MT = 2 activation rows (M = 2), each
    // chunk of weights is decoded once and feeds both rows; a second row past
    // M (M = 1 never takes MT = 2) would repeat row M - 1.
    typename F::Raw raw[R][TPW];
    constexpr int NX = XS ? 4 : 2;  // 16-byte loads per x chunk: 16 bf16, or 16 f32 to be scaled and rounded
    uint4 xr[TPW][MT][NX];
    const int t_last = max(0, min(t0 + nseg, a.T) - 1);
    // FP8: the wave's rows share one 128-row block, and its TPW segments need
    // 8 * TPW consecutive block scales: lanes load one each (one instruction
    // for the wave) and every chunk takes its scale from lane 8 u + lane / 8.
    // An index past the grid is clamped; only chunks past the last column,
    // whose results are discarded, would read it.
    float svec = 0.0f;
    if constexpr (KIND == kFp8)
        svec = a.grid[(min(r0, a.rows - 1) >> 7) * a.GC + min(t0 * 8 + lane, a.GC - 1)];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int q = min(min(t0 + u, t_last) * kLanes + lane, last_q);
        F::load_codes(a, r0, q, raw, u);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const uint4* xp = XS ? reinterpret_cast<const uint4*>(a.xs + (int64_t)q * kChunk)
                                 : reinterpret_cast<const uint4*>(a.x + (int64_t)min(m, a.M - 1) * a.K + (int64_t)q * kChunk);
#pragma unroll
            for (int h = 0; h < NX; ++h) xr[u][m][h] = xp[h];
        }
    }
    // Keep every load ahead of the arithmetic: with one shot of data per wave,
    // the bytes in flight per CU are what sets the streaming rate.
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (KIND == kFp8) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const float su = __shfl(svec, 8 * u + (lane >> 3));
#pragma unroll
            for (int i = 0; i < R; ++i) raw[i][u].s = su;
        }
    }
    float v[VP];
#pragma unroll
    for (int k = V; k < VP; ++k) v[k] = 0.0f;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const bool live = u < nseg && (t0 + u) * kLanes + lane <= last_q;
        float xf[MT][kChunk];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            if constexpr (XS) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    xf[m][4 * h + 0] = as_f32(bf16_of_scaled(a.xc, xr[u][m][h].x) << 16);
                    xf[m][4 * h + 1] = as_f32(bf16_of_scaled(a.xc, xr[u][m][h].y) << 16);
                    xf[m][4 * h + 2] = as_f32(bf16_of_scaled(a.xc, xr[u][m][h].z) << 16);
                    xf[m][4 * h + 3] = as_f32(bf16_of_scaled(a.xc, xr[u][m][h].w) << 16);
                }
            } else {
                widen8_bf16(xr[u][m][0], xf[m]);
                widen8_bf16(xr[u][m][1], xf[m] + 8);
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float w[kChunk];
            F::weights(raw[i][u], w, a.whole != 0);
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                float s = 0.0f;
#pragma unroll
                for (int j = 0; j < kChunk; ++j) s = __builtin_fmaf(w[j], xf[m][j], s);
                v[(i * TPW + u) * MT + m] = live ? s : 0.0f;
            }
        }
    }
    float red[VP / 4];
    tree64xV<VP>(v, red);
    // segment sum of (row i, segment u, activation row m): value k = (i * TPW + u) * MT + m
#define FP8BLK_P(i, u, m) \
    lane_value(red[(((i) * TPW + (u)) * MT + (m)) / 4], 16 * kRowOf4[(((i) * TPW + (u)) * MT + (m)) % 4])

    float y[R][MT];
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            y[i][m] = FP8BLK_P(i, 0, m);
#pragma unroll
            for (int u = 1; u < TPW; ++u)
                if (u < nseg) y[i][m] = y[i][m] + FP8BLK_P(i, u, m);
        }
    if (a.sw_log2 > 0) {
        if (lane == 0)
#pragma unroll
            for (int i = 0; i < R; ++i)
#pragma unroll
                for (int u = 0; u < TPW; ++u)
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        if (u < nseg) part[(((int64_t)rs * a.T + t0 + u) * R + i) * MT + m] = FP8BLK_P(i, u, m);
        __syncthreads();
        if (sp != 0) return;
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float* p = part + ((int64_t)rs * a.T * R + i) * MT + m;
                float v = p[0];
                for (int t = 1; t < a.T; ++t) v = v + p[t * R * MT];
                y[i][m] = v;
            }
    }
#undef FP8BLK_P
    // lane i * MT + m stores output (m, r0 + i)
    if (lane < R * MT) {
        const int i = lane / MT, m = lane % MT;
        float out = y[0][0];
#pragma unroll
        for (int ii = 0; ii < R; ++ii)
#pragma unroll
            for (int mm = 0; mm < MT; ++mm)
                if (lane == ii * MT + mm) out = y[ii][mm];
        if (m < a.M && r0 + i < a.rows) {
            a.y[(int64_t)m * a.rows + r0 + i] = out;
            if (a.xn) a.xn[r0 + i] = (uint16_t)bf16_of_scaled(a.xnc, as_u32(out));
        }
    }
}

// Up to kMaxGroup linears that share cols, x and M, in one launch: the
// workgroups of linear j are [start[j], start[j + 1]). Each output gets the
// same arithmetic as in a call of its own.
constexpr int kMaxGroup = 8;
struct GroupArgs {
    GemvArgs base;  // w, grid, y and rows are taken per linear
    const void* w[kMaxGroup];
    const float* grid[kMaxGroup];
    float* y[kMaxGroup];
    uint16_t* xn[kMaxGroup];  // per linear: the next input written beside y, or null
    int64_t rows[kMaxGroup];
    int64_t start[kMaxGroup + 1];
    int n;
};

__device__ __forceinline__ int group_of(const GroupArgs& g, int64_t block) {
    int j = 0;
    for (int k = 1; k < g.n; ++k)
        if (block >= g.start[k]) j = k;
    return j;
}

__host__ __device__ __forceinline__ GemvArgs group_args(const GroupArgs& g, int j) {
    GemvArgs a = g.base;
    a.w = g.w[j];
    a.grid = g.grid[j];
    a.y = g.y[j];
    a.xn = g.xn[j];
    a.rows = g.rows[j];
    return a;
}

template <int KIND, int R, int TPW, int MT>
__global__ __launch_bounds__(kThreads) void k_gemv_m1(const GemvArgs a) {
    m1_body<KIND, R, TPW, MT>(a, blockIdx.x);
}

template <int KIND, int R, int TPW, int MT>
__global__ __launch_bounds__(kThreads) void k_gemv_m1_group(const GroupArgs g) {
    const int j = __builtin_amdgcn_readfirstlane(group_of(g, blockIdx.x));
    m1_body<KIND, R, TPW, MT>(group_args(g, j), (int64_t)blockIdx.x - g.start[j]);
}

// The same kernels reading x as bf16(xc * xs) from an f32 vector (M = 1).
template <int R, int TPW>
__global__ __launch_bounds__(kThreads) void k_gemv_m1_scaled(const GemvArgs a) {
    m1_body<kFp8, R, TPW, 1, true>(a, blockIdx.x);
}

template <int R, int TPW>
__global__ __launch_bounds__(kThreads) void k_gemv_m1_group_scaled(const GroupArgs g) {
    const int j = __builtin_amdgcn_readfirstlane(group_of(g, blockIdx.x));
    m1_body<kFp8, R, TPW, 1, true>(group_args(g, j), (int64_t)blockIdx.x - g.start[j]);
}

template <int KIND, int MT, int R>
__global__ __launch_bounds__(kThreads) void k_panel(const GemvArgs a) {
    panel_body<KIND, MT, R>(a, blockIdx.x);
}

template <int KIND, int MT, int R>
__global__ __launch_bounds__(kThreads) void k_panel_group(const GroupArgs g) {
    const int j = __builtin_amdgcn_readfirstlane(group_of(g, blockIdx.x));
    panel_body<KIND, MT, R>(group_args(g, j), (int64_t)blockIdx.x - g.start[j]);
}

struct Plan {
    int MT, R, sw, tpw;  // tpw: compile-time segments per wave of the M = 1 kernel
    bool m1;             // the single-row kernel (else the panel kernel)
};

// Plan: a pure function of (rows, cols, M); it never changes bits.
// M = 1 and at most 16 segments: the one-shot kernel, TPW segments per wave
// and the rest of a row over sw waves (T <= TPW * sw):
// - T <= 2: TPW = T, R = 4 / TPW rows (four chunks per lane).
// - T >= 3 and fewer than 4096 rows: TPW = 4, R = 1. Small linears want the
//   most waves; measured on the whole-step sweep's launches, more chunks per
//   lane (fewer, longer waves) or fewer (more waves) are both slower.
// - T >= 3, 4096 rows or more: R = 2, which halves the activation chunks a
//   wave reads per weight chunk (every wave reads the x of its segments from
//   L2); TPW = 2 from 16384 rows when T <= 8, else 4. Measured, single cold
//   launches at cols 4096: 4096 rows 42.0% -> 43.2% of HBM peak, 12288 rows
//   60.9% -> 65.0%, 16384 rows 63.2% -> 67.6%, 129280 rows 75.7% -> 89.3%;
//   4096 x 16384 (split over 4 waves) 48.5% -> 56.7%.
// M = 2 and at most 4 segments: the same kernel with two activation rows
// (each weight chunk decoded once for both), the same R and TPW except TPW = 4
// from 4096 rows on. Measured, single cold launches at M = 2 against the
// panel kernel (same bits): 4096 x 4096 6.02 -> 5.71 us, 12288 x 4096 13.1 ->
// 11.5 us, 16384 x 4096 18.6 -> 15.1 us, 4096 x 2048 4.22 -> 3.96 us; with 16
// segments (4096 x 16384) the panel kernel stays faster, 19.1 against 21.0 us.
// Four activation rows in the one-shot kernel (M = 3, 4) measured slower than
// the panel kernel on every shape (12288 x 4096 at M = 4: 18.8-25.6 us over
// the row and segment splits against 17.2 us).
// Otherwise the panel kernel with R = 4 rows per wave, splitting the segments
// of a row over 2 or 4 waves while fewer than 4096 waves would run.
Plan make_plan(int64_t rows, int64_t K, int64_t M) {
    Plan p;
    const int64_t T = ceil_div(K, kSegCols);
    p.MT = M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16;
    if ((p.MT == 1 && T <= 16) || (p.MT == 2 && T <= 4)) {
        p.m1 = true;
        if (T <= 2) {
            p.tpw = (int)T;
            p.R = 4 / p.tpw;
        } else if (rows < 4096) {
            p.tpw = 4;
            p.R = 1;
        } else {
            p.tpw = p.MT == 1 && rows >= 16384 && T <= 8 ? 2 : 4;
            p.R = 2;
        }
        p.sw = T <= p.tpw ? 1 : T <= 2 * p.tpw ? 2 : 4;
        return p;
    }
    p.m1 = false;
    p.tpw = 0;
    p.R = 4;
    const int64_t groups = ceil_div(rows, p.R);
    p.sw = 1;
    while (p.sw < 4 && p.sw * 2 <= T && groups * p.sw < 4096) p.sw *= 2;
    return p;
}

int64_t blocks_for(const Plan& p, int64_t rows) { return ceil_div(ceil_div(rows, p.R), kWaves / p.sw); }

template <int KIND, int MT, int R>
void launch_panel(const GroupArgs& g, int64_t blocks, hipStream_t s) {
    constexpr int VP = R * MT < 4 ? 4 : R * MT;
    const int streams = kWaves / g.base.sw;
    const size_t lds = g.base.sw > 1 ? (size_t)streams * g.base.T * VP * sizeof(float) : 0;
    if (g.n == 1)
        k_panel<KIND, MT, R><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(group_args(g, 0));
    else
        k_panel_group<KIND, MT, R><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(g);
}

template <int KIND, int R, int TPW, int MT>
void launch_m1(const GroupArgs& g, int64_t blocks, hipStream_t s) {
    const int streams = kWaves / g.base.sw;
    const size_t lds = g.base.sw > 1 ? (size_t)streams * g.base.T * R * MT * sizeof(float) : 0;
    if constexpr (KIND == kFp8 && MT == 1) {
        if (g.base.xs) {
            if (g.n == 1)
                k_gemv_m1_scaled<R, TPW><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(group_args(g, 0));
            else
                k_gemv_m1_group_scaled<R, TPW><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(g);
            return;
        }
    }
    if (g.n == 1)
        k_gemv_m1<KIND, R, TPW, MT><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(group_args(g, 0));
    else
        k_gemv_m1_group<KIND, R, TPW, MT><<<dim3((unsigned)blocks), dim3(kThreads), lds, s>>>(g);
}

// One launch for g.n linears that share cols, x and M (g.w, g.grid, g.y and
// g.rows filled in). The plan is that of a single linear with all the rows.
template <int KIND>
int run(GroupArgs& g, int64_t cols, const uint16_t* x, int64_t M, hipStream_t s, const float* xs = nullptr,
        float xc = 1.0f) {
    int64_t all_rows = 0;
    for (int j = 0; j < g.n; ++j) all_rows += g.rows[j];
    const Plan p = make_plan(all_rows, cols, M);
    GemvArgs& a = g.base;
    a.w = nullptr;
    a.grid = nullptr;
    a.y = nullptr;
    a.rows = 0;
    a.x = x;
    a.xs = xs;
    a.xc = xc;
    a.xn = nullptr;
    a.K = (int)cols;
    a.M = (int)M;
    a.T = (int)ceil_div(cols, kSegCols);
    a.GC = (int)ceil_div(cols, kBlock);
    a.sw = p.sw;
    a.sw_log2 = p.sw == 4 ? 2 : p.sw == 2 ? 1 : 0;
    a.tpw = (int)ceil_div(a.T, p.sw);
    a.whole = KIND == kBf16 && cols % kSegCols == 0;
    g.start[0] = 0;
    for (int j = 0; j < g.n; ++j) g.start[j + 1] = g.start[j] + blocks_for(p, g.rows[j]);
    const int64_t blocks = g.start[g.n];
    if (blocks > 0x7fffffff) return FP8BLK_ERR_ARG;
    (void)hipGetLastError();
    if (p.m1) {
#define FP8BLK_M1(RR, TT, MM) \
    if (p.R == RR && p.tpw == TT && p.MT == MM) launch_m1<KIND, RR, TT, MM>(g, blocks, s)
        FP8BLK_M1(1, 4, 1); else FP8BLK_M1(2, 4, 1); else FP8BLK_M1(2, 2, 1); else FP8BLK_M1(4, 1, 1);
        else FP8BLK_M1(1, 4, 2); else FP8BLK_M1(2, 4, 2); else FP8BLK_M1(2, 2, 2); else FP8BLK_M1(4, 1, 2);
#undef FP8BLK_M1
    } else {
        switch (p.MT) {
            case 1: launch_panel<KIND, 1, 4>(g, blocks, s); break;
            case 2: launch_panel<KIND, 2, 4>(g, blocks, s); break;
            case 4: launch_panel<KIND, 4, 4>(g, blocks, s); break;
            case 8: launch_panel<KIND, 8, 4>(g, blocks, s); break;
            default: launch_panel<KIND, 16, 4>(g, blocks, s); break;
        }
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

template <int KIND>
int run_single(const void* w, const float* grid, int64_t rows, int64_t cols, const uint16_t* x, int64_t M,
               float* y, hipStream_t s) {
    GroupArgs g = {};
    g.n = 1;
    g.w[0] = w;
    g.grid[0] = grid;
    g.y[0] = y;
    g.rows[0] = rows;
    return run<KIND>(g, cols, x, M, s);
}

template <int KIND>
int run_grouped(const fp8blk_linear* lin, int n, int64_t cols, const uint16_t* x, int64_t M, hipStream_t s) {
    if (!lin || n < 1 || n > FP8BLK_MAX_GROUP) return FP8BLK_ERR_ARG;
    GroupArgs g = {};
    g.n = n;
    for (int j = 0; j < n; ++j) {
        const int st = check_common(lin[j].w, lin[j].rows, cols, x, M, lin[j].y, 0, nullptr, 0);
        if (st != FP8BLK_OK) return st;
        if (KIND == kFp8 && (!lin[j].scales_f32 || !aligned(lin[j].scales_f32, 4))) return FP8BLK_ERR_ARG;
        g.w[j] = lin[j].w;
        g.grid[j] = KIND == kFp8 ? lin[j].scales_f32 : nullptr;
        g.y[j] = lin[j].y;
        g.rows[j] = lin[j].rows;
    }
    return run<KIND>(g, cols, x, M, s);
}

// Whether the byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
    return pa < pb + nb && pb < pa + na;
}

// Scaled input: x = bf16(c * src) for one activation row, formed inside the
// single-row kernel's x loads. Only shapes that the single-row kernel takes
// at M = 1 (at most 16 segments) are accepted.
int run_scaled(const fp8blk_linear* lin, int n, int64_t cols, const float* src, float c, hipStream_t s) {
    if (!lin || n < 1 || n > FP8BLK_MAX_GROUP || !src || !aligned(src, 16) || ceil_div(cols, kSegCols) > 16)
        return FP8BLK_ERR_ARG;
    const uint16_t* xchk = reinterpret_cast<const uint16_t*>(src);  // for the common null / alignment checks
    GroupArgs g = {};
    g.n = n;
    for (int j = 0; j < n; ++j) {
        const int st = check_common(lin[j].w, lin[j].rows, cols, xchk, 1, lin[j].y, 0, nullptr, 0);
        if (st != FP8BLK_OK) return st;
        if (!lin[j].scales_f32 || !aligned(lin[j].scales_f32, 4)) return FP8BLK_ERR_ARG;
        g.w[j] = lin[j].w;
        g.grid[j] = lin[j].scales_f32;
        g.y[j] = lin[j].y;
        g.rows[j] = lin[j].rows;
        if (overlaps(src, (size_t)cols * sizeof(float), lin[j].y, (size_t)lin[j].rows * sizeof(float)))
            return FP8BLK_ERR_ARG;  // an output would overwrite the input it is read from
    }
    return run<kFp8>(g, cols, nullptr, 1, s, src, c);
}

// Next input: as run_grouped at M = 1, and linear k also writes
// x_next[r] = bf16(c * y_k[r]) beside its output (the input of a dependent
// linear that follows), in the single-row kernel's final stores.
int run_next(const fp8blk_linear* lin, int n, int64_t cols, const uint16_t* x, int k, float c, uint16_t* x_next,
             hipStream_t s) {
    if (!lin || n < 1 || n > FP8BLK_MAX_GROUP || k < 0 || k >= n || !x_next || !aligned(x_next, 2) ||
        ceil_div(cols, kSegCols) > 16)
        return FP8BLK_ERR_ARG;
    GroupArgs g = {};
    g.n = n;
    for (int j = 0; j < n; ++j) {
        const int st = check_common(lin[j].w, lin[j].rows, cols, x, 1, lin[j].y, 0, nullptr, 0);
        if (st != FP8BLK_OK) return st;
        if (!lin[j].scales_f32 || !aligned(lin[j].scales_f32, 4)) return FP8BLK_ERR_ARG;
        g.w[j] = lin[j].w;
        g.grid[j] = lin[j].scales_f32;
        g.y[j] = lin[j].y;
        g.rows[j] = lin[j].rows;
    }
    const size_t xn_bytes = (size_t)lin[k].rows * sizeof(uint16_t);
    if (overlaps(x_next, xn_bytes, x, (size_t)cols * sizeof(uint16_t))) return FP8BLK_ERR_ARG;
    for (int j = 0; j < n; ++j)
        if (overlaps(x_next, xn_bytes, lin[j].y, (size_t)lin[j].rows * sizeof(float))) return FP8BLK_ERR_ARG;
    g.xn[k] = x_next;
    g.base.xnc = c;
    return run<kFp8>(g, cols, x, 1, s);
}

static_assert(kMaxGroup == FP8BLK_MAX_GROUP, "group size of the ABI");

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
    return run_single<kFp8>(codes, scales_f32, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int bf16_gemv_twin(const uint16_t* w_bf16, int64_t rows, int64_t cols, const uint16_t* x_bf16,
                              int64_t M, float* y, void* ws, size_t ws_bytes, fp8blk_stream_t stream) {
    const int st = check_common(w_bf16, rows, cols, x_bf16, M, y,
                                fp8blk_workspace_bytes(FP8BLK_OP_BF16_TWIN, rows, cols, M), ws, ws_bytes);
    if (st != FP8BLK_OK) return st;
    return run_single<kBf16>(w_bf16, nullptr, rows, cols, x_bf16, M, y, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_gemv_grouped(const fp8blk_linear* linears, int n, int64_t cols, const uint16_t* x_bf16,
                                   int64_t M, fp8blk_stream_t stream) {
    return run_grouped<kFp8>(linears, n, cols, x_bf16, M, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int bf16_gemv_twin_grouped(const fp8blk_linear* linears, int n, int64_t cols, const uint16_t* x_bf16,
                                      int64_t M, fp8blk_stream_t stream) {
    return run_grouped<kBf16>(linears, n, cols, x_bf16, M, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_gemv_scaled_input(const uint8_t* codes, const float* scales_f32, int64_t rows, int64_t cols,
                                        const float* src_f32, float c, float* y, fp8blk_stream_t stream) {
    fp8blk_linear l;
    l.w = codes;
    l.scales_f32 = scales_f32;
    l.rows = rows;
    l.y = y;
    return run_scaled(&l, 1, cols, src_f32, c, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_gemv_grouped_scaled_input(const fp8blk_linear* linears, int n, int64_t cols,
                                                const float* src_f32, float c, fp8blk_stream_t stream) {
    return run_scaled(linears, n, cols, src_f32, c, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_gemv_next_input(const uint8_t* codes, const float* scales_f32, int64_t rows, int64_t cols,
                                      const uint16_t* x_bf16, float* y, float c, uint16_t* x_next,
                                      fp8blk_stream_t stream) {
    fp8blk_linear l;
    l.w = codes;
    l.scales_f32 = scales_f32;
    l.rows = rows;
    l.y = y;
    return run_next(&l, 1, cols, x_bf16, 0, c, x_next, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_gemv_grouped_next_input(const fp8blk_linear* linears, int n, int64_t cols,
                                              const uint16_t* x_bf16, int k, float c, uint16_t* x_next,
                                              fp8blk_stream_t stream) {
    return run_next(linears, n, cols, x_bf16, k, c, x_next, reinterpret_cast<hipStream_t>(stream));
}
