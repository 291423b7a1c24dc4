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
// matrix core always sees a 16-row panel (rows past M are filler whose outputs
// are dropped), and an output never depends on another row of the panel.
//
// What differs from fp8blk_gemv: the matrix core sums the 32 products of an
// instruction internally in an order the hardware does not document, so the
// result is not the documented f32 order of fp8blk_gemv and is checked against
// the exact sum by tolerance only.
//
// Order of operations for output (m, r): the columns are taken in windows of
// 128 (one scale-block column). Window w is four matrix instructions, (u, v) =
// (0,0), (0,1), (1,0), (1,1); instruction (u, v) takes from lane group kg
// (0..3) the 8 columns starting at 128 w + 32 kg + 16 u + 8 v, and all four
// accumulate into the same f32 tile. Windows are visited in increasing order
// inside each of the sw parts the windows are split into (part s covers
// windows [s * bpp, (s + 1) * bpp)); the sw partial tiles are added in part
// order. The split sw is a function of (rows, cols) only, never of M.
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

constexpr int kMfMinWaves = 4;   // waves of a workgroup: max(4, sw)
constexpr int kMfMaxWaves = 8;
constexpr int kMfMaxThreads = kMfMaxWaves * kLanes;
constexpr int kTile = 16;    // rows per matrix tile, and the padded panel
constexpr int kBufferWord3 = 0x00020000;    // buffer resource word 3 on gfx9-family targets: raw 32-bit data
constexpr uint32_t kPastEnd = 0x40000000u;  // a lane offset past a panel's end (panels are < 2 MB)

struct MfArgs {
    const void* w;        // uint8 codes or uint16 bf16 slab, [rows, K]
    const float* grid;    // f32 block scales (FP8 arm)
    const uint16_t* x;    // bf16 [M, K]
    float* y;             // f32 [M, rows]
    int64_t rows;
    int K, M, GC;
    int nwin;             // ceil(K / 128) column windows
    int sw_log2;          // waves splitting the windows of a row group: 1, 2, 4, 8
    int streams_log2;     // row groups per workgroup: log2(max(4, sw) / sw)
    int bpp;              // windows per part, ceil(nwin / sw)
};

// Window layout. The columns are taken in windows of 128 (one scale-block
// column); the matrix instruction wants tile row i (weights) and panel row n
// (activations) on lane bits 0..3 and a lane group kg = l >> 4 that is the
// same set of columns in both operands.
//
// Weights: for a 16-row tile, lane l loads from tile rows (l & 7) and 8 +
// (l & 7) the 16 codes of chunk l >> 3 of the window (columns [16 (l >> 3),
// +16)), so one load instruction covers 8 rows x 128 contiguous bytes. One
// exchange of lane bit 3 with the row-half register leaves tile row i = l & 15
// on lane bits 0..3: register u then holds, on lane (i, kg), row i, columns
// [32 kg + 16 u, +16).
//
// Activations: register (n1, n0) of lane l holds panel row 8 l3 + 4 l2 + 2 n1
// + n0 (lj = bit j of l), columns [8 G, 8 G + 8) with G = 8 l5 + 4 l4 + 2 l1 +
// l0: each group of four consecutive lanes reads 64 contiguous bytes of one
// row, and an instruction covers 4 rows x 256 bytes. Exchanging lane bit 0
// with n0 and lane bit 1 with n1 puts panel row n = l & 15 on lane bits 0..3;
// register (u, v) then holds, on lane (n, kg), row n, columns [32 kg + 16 u +
// 8 v, +8) -- the columns of half v of weight register u.

// Exchange lane bit B (B = 0, 1 or 3) with the register index of the pair
// (p, q): p'[l] = bit B of l ? q[l ^ 2^B] : p[l],
//         q'[l] = bit B of l ? q[l] : p[l ^ 2^B].
template <int B>
__device__ __forceinline__ uint32_t lane_flip(uint32_t v) {
    constexpr int ctrl = B == 0 ? kQuadXor1 : B == 1 ? kQuadXor2 : kRowRor8;  // lane ^ 2^B
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, ctrl, 0xF, 0xF, true);
}
template <int B>
__device__ __forceinline__ void exchange(uint4& p, uint4& q, bool hi) {
    uint32_t* pp = reinterpret_cast<uint32_t*>(&p);
    uint32_t* qq = reinterpret_cast<uint32_t*>(&q);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        if constexpr (B == 3) {
            swap_lane_bit3(pp[d], qq[d]);  // two bank-masked DPP moves, no selects
        } else {
            const uint32_t px = lane_flip<B>(pp[d]), qx = lane_flip<B>(qq[d]);
            const uint32_t np = hi ? qx : pp[d];
            const uint32_t nq = hi ? qq[d] : px;
            pp[d] = np;
            qq[d] = nq;
        }
    }
}

// The weights of one 16-row tile in one window, as loaded.
template <int KIND>
struct MfFetch;

template <>
struct MfFetch<0> {  // FP8: 16 codes per row half, decoded in registers
    struct Raw {
        uint4 c[2];  // [row half q]
    };
    // col: first column of the lane's chunk (already clamped into the row)
    __device__ __forceinline__ static void load(Raw& raw, const MfArgs& a, int64_t r_lo, int64_t r_hi, int col, bool,
                                                int) {
        const uint8_t* w = static_cast<const uint8_t*>(a.w);
        raw.c[0] = load_stream16(w + r_lo * a.K + col);
        raw.c[1] = load_stream16(w + r_hi * a.K + col);
    }
    // The four 8-wide operands, [u][v], after the exchange.
    __device__ __forceinline__ static void operands(Raw raw, float sc, bool hi, bool, v8bf op[2][2]) {
        exchange<3>(raw.c[0], raw.c[1], hi);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t d[4] = {raw.c[c].x, raw.c[c].y, raw.c[c].z, raw.c[c].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], sc, false);  // bytes 0, 1
                const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], sc, true);   // bytes 2, 3
                v8bf& o = op[c][k >> 1];
                o[4 * (k & 1) + 0] = p0[0];
                o[4 * (k & 1) + 1] = p0[1];
                o[4 * (k & 1) + 2] = p1[0];
                o[4 * (k & 1) + 3] = p1[1];
            }
        }
    }
};

// The bf16 slab: a lane's 16 columns are 32 bytes of its row. Loading its own
// two 16-byte halves would make each load instruction read every other 16
// bytes of the rows' 256-byte windows (half of every line it touches). In a
// full window, load 0 reads the first 128 bytes of the row and load 1 the
// second, lane chunk c = l / 8 taking 16-byte piece 2c (c < 4) or 2(c - 4) + 1
// (c >= 4), i.e. bytes +0 / +128 (c < 4) or -112 / +16 (c >= 4) from its own
// chunk; swap_lane_halves (lanes l and l + 32 hold chunks c and c + 4 of the
// same rows) then hands every lane its own two halves. A ragged last window
// keeps the per-lane loads (no swap).
__device__ __forceinline__ uint32_t twin_piece_shift(int lane) { return lane >= 32 ? (uint32_t)-112 : 0u; }

template <>
struct MfFetch<1> {  // bf16 slab: the same 16 columns are 32 bytes, two loads per row half
    struct Raw {
        uint4 c[2][2];  // [h][row half q]
    };
    // col: first column of the lane's chunk (already clamped into the row);
    // full: the window's 128 columns all exist (wave-uniform)
    __device__ __forceinline__ static void load(Raw& raw, const MfArgs& a, int64_t r_lo, int64_t r_hi, int col,
                                                bool full, int lane) {
        const char* w = static_cast<const char*>(a.w);
        const uint32_t d0 = full ? twin_piece_shift(lane) : 0u, d1 = full ? d0 + 128u : 16u;
        const char* lo = w + (r_lo * a.K + col) * 2;
        const char* hi = w + (r_hi * a.K + col) * 2;
        raw.c[0][0] = load_stream16(lo + (int32_t)d0);
        raw.c[1][0] = load_stream16(lo + (int32_t)d1);
        raw.c[0][1] = load_stream16(hi + (int32_t)d0);
        raw.c[1][1] = load_stream16(hi + (int32_t)d1);
    }
    __device__ __forceinline__ static void operands(Raw raw, float, bool hi, bool full, v8bf op[2][2]) {
        if (full) {
            swap_lane_halves(raw.c[0][0], raw.c[1][0]);
            swap_lane_halves(raw.c[0][1], raw.c[1][1]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            exchange<3>(raw.c[h][0], raw.c[h][1], hi);
            op[0][h] = __builtin_bit_cast(v8bf, raw.c[h][0]);
            op[1][h] = __builtin_bit_cast(v8bf, raw.c[h][1]);
        }
    }
};

// Everything one window needs, loaded ahead of the matrix work that uses it.
// XR activation registers are loaded: 1 for M = 1, 2 for M = 2, else 4 (the
// others would hold only panel rows >= M).
template <int KIND, int TILES, int XR>
struct MfWindow {
    typename MfFetch<KIND>::Raw w[TILES];
    uint4 x[4];  // [2 n1 + n0] as loaded, [2 u + v] after the exchanges
    float sc;
};

// Per-lane constants of the layout.
struct MfLane {
    int64_t r0;         // first row of the wave
    int r;              // l & 7
    int wchunk;         // 16 (l >> 3)
    int xcol;           // 8 G
    uint32_t xrow[4];   // byte offset of panel row 8 l3 + 4 l2 + 2 n1 + n0 in x; kPastEnd for rows >= M
    bool b0, b1, b3;    // lane bits 0, 1, 3
    int lane;
};

// What one window of a single call needs: the tiles' weights, the panel
// window, and each tile's block scale (a wave's tiles may lie in two 128-row
// scale blocks when it takes three of them).
template <int KIND, int TILES, int XR>
struct MfCallWindow {
    typename MfFetch<KIND>::Raw w[TILES];
    uint4 x[4];  // [2 n1 + n0] as loaded, [2 u + v] after the exchanges
    float sc[TILES];
};

typedef __attribute__((address_space(4))) const float constant_f32;

// The activations come through a buffer resource over the panel: a lane whose
// panel row is >= M has an offset past the panel's end, and the range check
// returns zeros without touching memory (at M = 1, three lanes in four; at
// M = 8, half), so a short panel costs only its own bytes.
template <int KIND, int TILES, int XR>
__device__ __forceinline__ void mf_issue(MfCallWindow<KIND, TILES, XR>& b, const MfArgs& a, const MfLane& L,
                                         __amdgpu_buffer_rsrc_t xr, int win) {
    const int base = win * kBlock;
    const int wcol = min(base + L.wchunk, a.K - 16);  // a chunk past the last column re-reads the last one
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int64_t lo = min(L.r0 + t * kTile + L.r, a.rows - 1);
        const int64_t hi = min(L.r0 + t * kTile + 8 + L.r, a.rows - 1);
        MfFetch<KIND>::load(b.w[t], a, lo, hi, wcol, base + kBlock <= a.K, L.lane);
    }
    const uint32_t xc = (uint32_t)(min(base + L.xcol, a.K - 8) - base) * 2;
#pragma unroll
    for (int k = 0; k < XR; ++k) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(L.xrow[k] + xc), base * 2, 0);
        b.x[k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        b.sc[t] = 1.0f;
        if constexpr (KIND == 0) b.sc[t] = *(constant_f32*)(a.grid + (min(L.r0 + t * kTile, a.rows - 1) >> 7) * a.GC + win);
    }
}

template <int KIND, int TILES, int XR>
__device__ __forceinline__ void mf_compute(MfCallWindow<KIND, TILES, XR> b, const MfArgs& a, const MfLane& L, int win,
                                           v4f* acc) {
    const int base = win * kBlock;
    if (base + kBlock > a.K && base + L.xcol + 8 > a.K) {
        // ragged last window: activation columns past the end feed zeros
#pragma unroll
        for (int k = 0; k < XR; ++k) b.x[k] = make_uint4(0, 0, 0, 0);
    }
    // registers not loaded hold only panel rows >= M: any values serve, their outputs are not stored
#pragma unroll
    for (int k = XR; k < 4; ++k) b.x[k] = b.x[0];
    exchange<0>(b.x[0], b.x[1], L.b0);
    exchange<0>(b.x[2], b.x[3], L.b0);
    exchange<1>(b.x[0], b.x[2], L.b1);
    exchange<1>(b.x[1], b.x[3], L.b1);
    // every tile's operands first, then the matrix instructions with the tile
    // innermost (independent accumulator chains); each tile still takes
    // (u, v) = (0,0), (0,1), (1,0), (1,1) in that order
    v8bf op[TILES][2][2];
#pragma unroll
    for (int t = 0; t < TILES; ++t) MfFetch<KIND>::operands(b.w[t], b.sc[t], L.b3, base + kBlock <= a.K, op[t]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int t = 0; t < TILES; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][u][v], __builtin_bit_cast(v8bf, b.x[2 * u + v]),
                                                                 acc[t], 0, 0, 0);
}

// After the windows: the sw parts of a row group meet in LDS and the wave of
// part 0 adds them in part order; then lane l writes D[4 (l / 16) + e][l % 16]
// (row 4 (l / 16) + e of the tile, panel row l % 16).
template <int TILES>
__device__ __forceinline__ void mf_finish(const MfArgs& a, const MfLane& L, int wave, int sp, v4f* acc,
                                          v4f (*part)[TILES][kLanes]) {
    const int lane = L.lane;
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
    const int n = lane & 15, kg = lane >> 4;
    if (n < a.M) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int64_t r = L.r0 + t * kTile + 4 * kg + e;
                if (r < a.rows) a.y[(int64_t)n * a.rows + r] = acc[t][e];
            }
    }
}

template <int TILES>
__device__ __forceinline__ MfLane mf_lane(const MfArgs& a, int wave, int lane) {
    const int rs = wave >> a.sw_log2;
    MfLane L;
    L.r0 = (((int64_t)blockIdx.x << a.streams_log2) + rs) * (TILES * kTile);
    L.r = lane & 7;
    L.wchunk = 16 * (lane >> 3);
    L.xcol = 8 * (((lane >> 4) << 2) | (lane & 3));
    const int xr_base = 8 * ((lane >> 3) & 1) + 4 * ((lane >> 2) & 1);
#pragma unroll
    for (int k = 0; k < 4; ++k) L.xrow[k] = xr_base + k < a.M ? (uint32_t)((xr_base + k) * a.K * 2) : kPastEnd;
    L.b0 = (lane & 1) != 0;
    L.b1 = (lane & 2) != 0;
    L.b3 = (lane & 8) != 0;
    L.lane = lane;
    return L;
}

// A wave owns TILES tiles of 16 consecutive rows and one part of the windows;
// the loads of the next DEPTH - 1 windows are in flight while a window is
// multiplied. Loads are unconditional: past the end of the part they re-read
// its last window, which is then not used.
template <int KIND, int TILES, int XR, int DEPTH>
__global__ __launch_bounds__(kMfMaxThreads) void k_mfma(const MfArgs a) {
    using Win = MfCallWindow<KIND, TILES, XR>;
    __shared__ v4f part[kMfMaxWaves][TILES][kLanes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int sp = wave & ((1 << a.sw_log2) - 1);
    const MfLane L = mf_lane<TILES>(a, wave, lane);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), (short)0, a.M * a.K * 2, kBufferWord3);
    const int wb = sp * a.bpp;
    const int we = min(a.nwin, wb + a.bpp);

    v4f acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (wb < we) {
        Win buf[DEPTH];
#pragma unroll
        for (int d = 0; d + 1 < DEPTH; ++d) mf_issue(buf[d], a, L, xr, min(wb + d, we - 1));
        for (int w = wb; w < we; w += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; ++d) {
                mf_issue(buf[(d + DEPTH - 1) % DEPTH], a, L, xr, min(w + d + DEPTH - 1, we - 1));
                __builtin_amdgcn_sched_barrier(0);
                if (w + d < we) mf_compute(buf[d], a, L, w + d, acc);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    mf_finish<TILES>(a, L, wave, sp, acc, part);
}

// One shot: every load of a wave's part (at most NW windows) is issued before
// any matrix work, so that a compute unit has its whole share of a cold
// linear in flight at once; a single launch is then bound by how fast HBM
// answers, not by how many loads each wave keeps waiting. A part shorter
// than NW re-reads its last window for the missing ones (not used). WAVES is
// the workgroup's wave count, which sets the register budget.
template <int KIND, int TILES, int XR, int NW, int WAVES>
__global__ __launch_bounds__(WAVES * kLanes) void k_mfma_shot(const MfArgs a) {
    using Win = MfCallWindow<KIND, TILES, XR>;
    __shared__ v4f part[WAVES][TILES][kLanes];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const int sp = wave & ((1 << a.sw_log2) - 1);
    const MfLane L = mf_lane<TILES>(a, wave, lane);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.x), (short)0, a.M * a.K * 2, kBufferWord3);
    const int wb = sp * a.bpp;
    const int we = min(a.nwin, wb + a.bpp);

    v4f acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    if (wb < we) {
        Win buf[NW];
#pragma unroll
        for (int d = 0; d < NW; ++d) mf_issue(buf[d], a, L, xr, min(wb + d, we - 1));
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int d = 0; d < NW; ++d)
            if (wb + d < we) mf_compute(buf[d], a, L, wb + d, acc);
    }
    mf_finish<TILES>(a, L, wave, sp, acc, part);
}

// Plan. The split sw is a function of (rows, cols) only -- it fixes the
// order of the sums -- : the largest of 1, 2, 4, 8 that leaves >= 8 windows
// per part, or >= 4 windows while fewer than 1024 single-tile waves would run.
// TILES only changes which wave computes an output, not its order, so it may
// follow the device: a wave takes the most row tiles (up to 4) that still
// leave at least one workgroup per compute unit. Row tiles in one wave share
// its activation loads, and the activations, not the weights, are what a
// wave's loads mostly carry from a 4-row panel on (16 panel rows x 128
// columns of bf16 per window, against 16 rows x 128 codes per tile); but a
// compute unit without a workgroup reads nothing. On 12288 x 4096 this is 3
// tiles (256 workgroups): 42 -> 50% of HBM peak at M = 16, 45 -> 53% at
// M = 8, against 4 tiles (192 workgroups, a quarter of the compute units
// idle) and 1 tile (768 workgroups, three times the activation loads).
// The loads are issued in one shot (nw = windows per part, FP8 arm) where a
// part is 2, 4 or 8 windows, M <= 8, and either M <= 2 or the waves take one
// tile anyway: a wave then has all of its part in flight at once instead of
// two windows. Measured on cold single launches (same bits): M = 1 on
// 4096 x 4096 6.5 -> 5.4 us, 16384 x 4096 15.8 -> 14.2 us, 12288 x 4096 11.6
// -> 11.3 us, 1024 x 4096 4.9 -> 4.65 us; M = 8 on 4096 x 4096 7.0 -> 6.8 us.
// With more activation rows and several tiles per wave the two-deep pipeline
// stays faster (12288 x 4096 at M = 8: 11.6 us against 13.3), and at M = 16
// too (4096 x 4096: 7.25 against 7.6).
struct MfPlan {
    int tiles, sw, nw;  // nw: windows per wave loaded in one shot (0: the two-deep pipeline)
};
MfPlan mf_plan(int64_t rows, int64_t K, int64_t M, int cus, bool fp8) {
    MfPlan p;
    const int64_t nwin = ceil_div(K, (int64_t)kBlock);
    const int64_t groups1 = ceil_div(rows, (int64_t)kTile);
    p.sw = 1;
    while (p.sw < kMfMaxWaves && (nwin >= 16 * p.sw || (nwin >= 8 * p.sw && groups1 * p.sw < 1024))) p.sw *= 2;
    const int streams = (p.sw >= kMfMinWaves ? p.sw : kMfMinWaves) / p.sw;  // row groups per workgroup
    p.tiles = 1;
    for (int t = 4; t > 1; --t)
        if (ceil_div(ceil_div(groups1, (int64_t)t), (int64_t)streams) >= cus) {
            p.tiles = t;
            break;
        }
    const int64_t bpp = ceil_div(nwin, (int64_t)p.sw);
    p.nw = 0;
    if (fp8 && (bpp == 2 || bpp == 4 || bpp == 8) && M <= 8 && (M <= 2 || p.tiles == 1)) {
        p.nw = (int)bpp;
        p.tiles = 1;
    }
    return p;
}

template <int KIND, int XR>
void mf_launch(const MfPlan& p, dim3 nb, dim3 nt, hipStream_t s, const MfArgs& a) {
    if constexpr (KIND == 0) {
        if (p.nw > 0) {
            const bool w4 = nt.x == 4 * kLanes;
            switch (p.nw) {
                case 8:
                    if (w4) k_mfma_shot<0, 1, XR, 8, 4><<<nb, nt, 0, s>>>(a);
                    else k_mfma_shot<0, 1, XR, 8, 8><<<nb, nt, 0, s>>>(a);
                    return;
                case 4:
                    if (w4) k_mfma_shot<0, 1, XR, 4, 4><<<nb, nt, 0, s>>>(a);
                    else k_mfma_shot<0, 1, XR, 4, 8><<<nb, nt, 0, s>>>(a);
                    return;
                default:
                    if (w4) k_mfma_shot<0, 1, XR, 2, 4><<<nb, nt, 0, s>>>(a);
                    else k_mfma_shot<0, 1, XR, 2, 8><<<nb, nt, 0, s>>>(a);
                    return;
            }
        }
    }
    switch (p.tiles) {
        case 4: k_mfma<KIND, 4, XR, 2><<<nb, nt, 0, s>>>(a); break;
        case 3: k_mfma<KIND, 3, XR, 2><<<nb, nt, 0, s>>>(a); break;
        case 2: k_mfma<KIND, 2, XR, 2><<<nb, nt, 0, s>>>(a); break;
        default: k_mfma<KIND, 1, XR, 2><<<nb, nt, 0, s>>>(a); break;
    }
}

template <int KIND>
int mf_run(const void* w, const float* grid, int64_t rows, int64_t cols, const uint16_t* x, int64_t M, float* y,
           hipStream_t s) {
    const int cus = device_cus();
    if (cus <= 0) return FP8BLK_ERR_HIP;
    const MfPlan p = mf_plan(rows, cols, M, cus, KIND == 0);
    MfArgs a;
    a.w = w;
    a.grid = grid;
    a.x = x;
    a.y = y;
    a.rows = rows;
    a.K = (int)cols;
    a.M = (int)M;
    a.GC = (int)ceil_div(cols, kBlock);
    a.nwin = a.GC;
    a.sw_log2 = p.sw == 8 ? 3 : p.sw == 4 ? 2 : p.sw == 2 ? 1 : 0;
    const int waves = p.sw > kMfMinWaves ? p.sw : kMfMinWaves;
    a.streams_log2 = p.sw >= kMfMinWaves ? 0 : a.sw_log2 == 1 ? 1 : 2;
    a.bpp = (int)ceil_div(a.nwin, p.sw);
    const int streams = waves / p.sw;
    const int64_t blocks = ceil_div(ceil_div(rows, (int64_t)kTile * p.tiles), streams);
    if (blocks > 0x7fffffff) return FP8BLK_ERR_ARG;
    (void)hipGetLastError();
    const dim3 nb((unsigned)blocks), nt(waves * kLanes);
    if (M > 2)
        mf_launch<KIND, 4>(p, nb, nt, s, a);
    else if (M == 2)
        mf_launch<KIND, 2>(p, nb, nt, s, a);
    else
        mf_launch<KIND, 1>(p, nb, nt, s, a);
    return launch_status();
}

// ---------------------------------------------------------------------------
// Matrix-core sequence: a list of independent linears with a panel of M rows
// each, run by one persistent kernel. A unit is TILES 16-row tiles of one
// linear (inside one 128-row scale block) across all its column windows, in
// increasing window order into one accumulator per tile (the order of
// k_mfma with one part). Units are numbered over the list in order; wave w of
// W takes units w, w + W, ...; each wave loads the next window (of this unit
// or of its next one) before it multiplies the current one.

struct alignas(64) MfSeqLin {
    const void* w;       // codes or bf16 slab [rows, K]
    const float* grid;   // f32 block scales (FP8 arm)
    const uint16_t* x;   // bf16 [M, K]
    float* y;            // f32 [M, rows]
    int64_t rows;
    int32_t K, M, GC, nwin;
    int32_t vec_store;   // 1: y is 16-byte aligned and rows % 4 == 0 (each panel row's outputs store 4 at a time)
    int32_t pad;
};
static_assert(sizeof(MfSeqLin) == kSeqDescBytes, "descriptor size of the plan");

// Row tiles per unit: 4 for panels of 8 rows or more (the tiles share a
// wave's activation loads), else 2. Measured on the whole-step sweep.
constexpr int mf_seq_tiles(int M) { return M >= 8 ? 4 : 2; }

// Per-unit addressing, computed once when a wave starts a unit: wave-uniform
// bases plus 32-bit lane offsets, so that a window's loads need no vector
// arithmetic (the row clamps of the last, partial tile group are folded into
// the offsets).
template <int TILES, int XR>
struct MfUnit {
    const char* w;              // weights of the unit's first row
    const char* x;              // the linear's activation panel
    int32_t x_bytes;            // its bytes, M * K * 2
    const float* g;             // the unit's row of block scales (FP8 arm)
    uint32_t roff[TILES][2];    // lane: byte offset of its rows (lo, hi) + its chunk's first column
    uint32_t xoff[XR];          // lane: byte offset of its panel rows + its column group (kPastEnd: rows >= M)
};

struct MfPos {
    int64_t u, v;  // unit (list numbering) and unit within its linear
    int win, j;
    bool more;     // false: past the wave's last window (the position repeats the last one)
    MfSeqLin d;
};

template <int KIND, int TILES, int XR>
__device__ __forceinline__ void mf_unit(MfUnit<TILES, XR>& U, const MfSeqLin& d, int64_t v, int lane) {
    constexpr int E = KIND == 0 ? 1 : 2;
    const int64_t r0 = v * (TILES * kTile);
    U.w = static_cast<const char*>(d.w) + r0 * d.K * E;
    U.x = reinterpret_cast<const char*>(d.x);
    U.x_bytes = d.M * d.K * 2;
    U.g = d.grid + (r0 >> 7) * d.GC;
    const int r = lane & 7, wchunk = 16 * (lane >> 3);
#pragma unroll
    for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t row = min(r0 + t * kTile + 8 * h + r, d.rows - 1) - r0;
            U.roff[t][h] = (uint32_t)((row * d.K + wchunk) * E);
        }
    const int xr_base = 8 * ((lane >> 3) & 1) + 4 * ((lane >> 2) & 1);
    const int xcol = 8 * (((lane >> 4) << 2) | (lane & 3));
#pragma unroll
    // Panel rows >= M are never stored: their lanes take an offset past the
    // panel's end, and the buffer range check gives zeros without a memory
    // access (at M <= 4, three of every four lanes; at M = 8, half).
    for (int k = 0; k < XR; ++k)
        U.xoff[k] = xr_base + k < d.M ? (uint32_t)(((xr_base + k) * d.K + xcol) * 2) : kPastEnd;
}

__device__ __forceinline__ MfPos mf_next(const MfPos& p, const MfSeqLin* lin, const int64_t* pre, int64_t W,
                                         int64_t total) {
    MfPos n = p;
    if (!p.more) return n;
    if (p.win + 1 < p.d.nwin) {
        n.win = p.win + 1;
    } else if (p.u + W < total) {
        n.u = p.u + W;
        n.v = p.v + W;
        n.win = 0;
        if (n.u >= pre[n.j + 1]) {
            do ++n.j;
            while (n.u >= pre[n.j + 1]);
            n.d = lin[n.j];
            n.v = n.u - pre[n.j];
        }
    } else {
        n.more = false;
    }
    return n;
}


// The loads of window `win` of a unit: the unit's bases plus the lane
// offsets. In the last window of a row whose cols is not a multiple of 128,
// a lane whose chunk lies past the last column moves back to the last chunk
// (its products are then multiplied by the zeroed activations, see
// mf_seq_compute); elsewhere the shift is 0. No branch: every window issues
// the same loads, so the waits for a window never cover the next one's. The
// block scale is the same for every lane: one scalar load.
template <int KIND, int TILES, int XR>
__device__ __forceinline__ void mf_seq_issue(MfWindow<KIND, TILES, XR>& b, const MfUnit<TILES, XR>& U, int K, int win,
                                             int lane) {
    constexpr int E = KIND == 0 ? 1 : 2;
    const int base = win * kBlock;
    const char* wsrc = U.w + base * E;
    const int wchunk = 16 * (lane >> 3), xcol = 8 * (((lane >> 4) << 2) | (lane & 3));
    const uint32_t wshift = (uint32_t)((min(base + wchunk, K - 16) - base - wchunk) * E);  // 0, or minus the overrun
    const uint32_t xshift = (uint32_t)((min(base + xcol, K - 8) - base - xcol) * 2);
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const uint32_t lo = U.roff[t][0] + wshift, hi = U.roff[t][1] + wshift;
        if constexpr (KIND == 0) {
            b.w[t].c[0] = load_stream16(wsrc + lo);
            b.w[t].c[1] = load_stream16(wsrc + hi);
        } else {
            // contiguous pieces in a full window (see MfFetch<1>); not with 4
            // tiles, whose registers could then hold only one wave per SIMD
            const bool full = TILES < 4 && base + kBlock <= K;
            const uint32_t d0 = full ? twin_piece_shift(lane) : 0u, d1 = full ? d0 + 128u : 16u;
            b.w[t].c[0][0] = load_stream16(wsrc + (uint32_t)(lo + d0));
            b.w[t].c[1][0] = load_stream16(wsrc + (uint32_t)(lo + d1));
            b.w[t].c[0][1] = load_stream16(wsrc + (uint32_t)(hi + d0));
            b.w[t].c[1][1] = load_stream16(wsrc + (uint32_t)(hi + d1));
        }
    }
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(U.x), (short)0, U.x_bytes, kBufferWord3);
#pragma unroll
    for (int k = 0; k < XR; ++k) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(U.xoff[k] + xshift), base * 2, 0);
        b.x[k] = make_uint4(v[0], v[1], v[2], v[3]);
    }
    b.sc = 1.0f;
    if constexpr (KIND == 0) b.sc = *(constant_f32*)(U.g + win);
}

template <int KIND, int TILES, int XR>
__device__ __forceinline__ void mf_seq_compute(MfWindow<KIND, TILES, XR> b, int K, int win, int lane, v4f* acc) {
    const int base = win * kBlock;
    const int xcol = 8 * (((lane >> 4) << 2) | (lane & 3));
    if (base + kBlock > K && base + xcol + 8 > K) {
        // ragged last window: activation columns past the end feed zeros
#pragma unroll
        for (int k = 0; k < XR; ++k) b.x[k] = make_uint4(0, 0, 0, 0);
    }
    // registers not loaded hold only panel rows >= M: any values serve, their outputs are not stored
#pragma unroll
    for (int k = XR; k < 4; ++k) b.x[k] = b.x[0];
    const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0, b3 = (lane & 8) != 0;
    exchange<0>(b.x[0], b.x[1], b0);
    exchange<0>(b.x[2], b.x[3], b0);
    exchange<1>(b.x[0], b.x[2], b1);
    exchange<1>(b.x[1], b.x[3], b1);
    // Every tile's operands first, then the matrix instructions with the tile
    // innermost: the TILES accumulator chains are independent, so each
    // instruction waits on one issued TILES instructions earlier. Each tile
    // still takes (u, v) = (0,0), (0,1), (1,0), (1,1) in that order.
    v8bf op[TILES][2][2];
#pragma unroll
    for (int t = 0; t < TILES; ++t) MfFetch<KIND>::operands(b.w[t], b.sc, b3, TILES < 4 && base + kBlock <= K, op[t]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int v = 0; v < 2; ++v)
#pragma unroll
            for (int t = 0; t < TILES; ++t)
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op[t][u][v], __builtin_bit_cast(v8bf, b.x[2 * u + v]),
                                                                 acc[t], 0, 0, 0);
}

// Lane (n, kg) = (l % 16, l / 16) holds D[4 kg + e][n], e = 0..3: rows
// 4 kg .. 4 kg + 3 of the tile for panel row n, four consecutive outputs of
// y[n]. yu points at y[0][first row of the unit], `rows` is the row stride of
// y and `left` the rows of the unit that exist (rows - first row, at most
// TILES * 16). When vec is set (the linear allows it) four outputs leave as
// one 16-byte store (a tile is one store instruction writing 16 panel rows x
// 64 bytes, half of a 128-byte line each; the next tile writes the other
// half), else one by one. The stores go through L2, which merges the two
// halves of a line before it reaches HBM: with the nontemporal hint each half
// went out on its own and HBM took 28% more bytes than the outputs hold at
// M = 16 (71.8 MB written against 56.2 MB; plain stores: 56.2 MB), for no
// gain in time.
template <int TILES>
__device__ __forceinline__ void mf_seq_store_at(float* yu, int64_t rows, int left, bool vec, int M, int lane,
                                                const v4f* acc) {
    const int n = lane & 15, kg = lane >> 4;
    if (n >= M) return;
    float* yrow = yu + (int64_t)n * rows;
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
        const int r = t * kTile + 4 * kg;
        if (vec && r + 3 < left) {
            typedef __attribute__((address_space(1))) v4f global_v4f;
            *(global_v4f*)(yrow + r) = acc[t];
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (r + e < left) store_global_f32(yrow + r + e, acc[t][e]);
        }
    }
}

// Where a finished unit's outputs go. A stream of reads runs markedly slower
// while writes are mixed into it than when the same bytes are written in one
// burst after it (measured with a bare 3 GiB read by 2048 waves: 1 KB written
// per 64 KB read costs 13% of the read rate, the same bytes written at each
// wave's end 6%). With a panel of 8 or more rows the outputs are 1/57 (M = 16)
// of the bytes read, so each wave keeps the outputs of its first units in its
// own part of the workgroup's LDS (on the FP8 arm the next PARK in registers)
// and writes them after its last unit; units past that are written when they
// finish. Smaller panels write when each unit finishes. Only where and when
// the outputs are stored changes, never their values.
//
// An LDS slot holds one unit: lane (n, kg) with n < M puts tile t's four
// outputs at 16 ((t M + n) 4 + kg) bytes. Where unit k goes is recorded in
// lane k of five registers (its y address, y's row stride, and its row count
// with the vector-store flag), so the final writes need no loads but LDS.
constexpr int kMfSeqLdsBytes = 80 * 1024;                       // per workgroup: at most 2 per compute unit
constexpr int kMfSeqWaveLds = kMfSeqLdsBytes / kSeqWaves;       // per wave
constexpr int kMfSeqHoldMinM = 8;                               // smallest panel whose outputs are held back
static_assert(kMfSeqBlocksPerCU * kMfSeqLdsBytes <= 160 * 1024 && (kMfSeqBlocksPerCU + 1) * kMfSeqLdsBytes > 160 * 1024,
              "the LDS of a workgroup caps a compute unit at kMfSeqBlocksPerCU of them");

static_assert(mf_seq_blocks_per_cu(true, kMfSeqHoldMinM) == kMfSeqBlocksPerCU &&
                  mf_seq_blocks_per_cu(false, 1) == kMfSeqBlocksPerCU,
              "panels whose outputs are held, and the bf16 arm, run two workgroups per compute unit");

struct MfOut {
    unsigned char* lds;  // the wave's part of the workgroup's LDS
    int M;               // panel rows of the list (the plan's; every descriptor holds the same)
    int slot_bytes;      // TILES * M * 64
    int slots;           // units the LDS part holds (0 below kMfSeqHoldMinM)
    int k;               // units finished so far
    uint32_t y_lo, y_hi, rows_lo, rows_hi, left_vec;  // lane k: record of held unit k
};

template <int TILES, int PARK>
struct MfPark {
    v4f acc[PARK > 0 ? PARK : 1][TILES];  // acc[i]: held unit slots + i
};

template <int TILES>
__device__ __forceinline__ void mf_seq_store(const MfSeqLin& d, int64_t v, int lane, const v4f* acc) {
    const int64_t r0 = v * (TILES * kTile);
    mf_seq_store_at<TILES>(d.y + r0, d.rows, (int)min(d.rows - r0, (int64_t)(TILES * kTile)), d.vec_store != 0, d.M,
                           lane, acc);
}

// Outputs are held back only with 4-tile units, the units of panels of
// kMfSeqHoldMinM rows or more; the smaller panels' kernels leave the holding
// code out.
template <int TILES>
constexpr bool mf_seq_holds() { return TILES == mf_seq_tiles(kMfSeqHoldMinM); }

template <int TILES, int PARK>
__device__ __forceinline__ void mf_seq_retire(const MfSeqLin& d, int64_t v, int lane, const v4f* acc, MfOut& o,
                                              MfPark<TILES, PARK>& park) {
    if (mf_seq_holds<TILES>() && o.k < o.slots + PARK) {
        const int64_t r0 = v * (TILES * kTile);
        const uint64_t yu = reinterpret_cast<uint64_t>(d.y + r0);
        const uint32_t lv = (uint32_t)min(d.rows - r0, (int64_t)(TILES * kTile)) | (d.vec_store ? 0x10000u : 0u);
        const bool mine = lane == o.k;  // lane k keeps unit k's record
        o.y_lo = mine ? (uint32_t)yu : o.y_lo;
        o.y_hi = mine ? (uint32_t)(yu >> 32) : o.y_hi;
        o.rows_lo = mine ? (uint32_t)d.rows : o.rows_lo;
        o.rows_hi = mine ? (uint32_t)((uint64_t)d.rows >> 32) : o.rows_hi;
        o.left_vec = mine ? lv : o.left_vec;
        if (o.k < o.slots) {
            const int n = lane & 15, kg = lane >> 4;
            if (n < o.M) {
                unsigned char* slot = o.lds + o.k * o.slot_bytes;
#pragma unroll
                for (int t = 0; t < TILES; ++t) *reinterpret_cast<v4f*>(slot + ((t * o.M + n) * 4 + kg) * 16) = acc[t];
            }
        } else {
#pragma unroll
            for (int i = 0; i < PARK; ++i)
                if (o.k == o.slots + i)
#pragma unroll
                    for (int t = 0; t < TILES; ++t) park.acc[i][t] = acc[t];
        }
    } else {
        mf_seq_store<TILES>(d, v, lane, acc);
    }
    ++o.k;
}

// Held unit k's outputs, from its LDS slot, written so that every store
// instruction covers whole 128-byte lines of y: instruction i takes panel rows
// 4i .. 4i + 3; lane l carries piece p = l % 16 (rows 4p .. 4p + 3 of the
// unit: tile p / 4, lane group p % 4) of panel row 4i + l / 16. A unit's 64
// outputs of a panel row are then 256 contiguous bytes from 16 lanes of one
// instruction, so the nontemporal stores (0.5 point faster than plain ones at
// M = 16) reach HBM as whole lines: 56.2 MB written at M = 16, the outputs'
// own bytes. (With the register layout, each store writes half lines and the
// nontemporal ones went out as 71.8 MB.)
template <int TILES>
__device__ __forceinline__ void mf_seq_store_slot(const MfOut& o, int k, const unsigned char* slot, int lane) {
    static_assert(TILES * 4 == 16, "a held unit is 64 rows: 16 pieces of 4 outputs per panel row");
    const uint64_t yu = ((uint64_t)__builtin_amdgcn_readlane(o.y_hi, k) << 32) | (uint32_t)__builtin_amdgcn_readlane(o.y_lo, k);
    const int64_t rows = (int64_t)(((uint64_t)__builtin_amdgcn_readlane(o.rows_hi, k) << 32) |
                                   (uint32_t)__builtin_amdgcn_readlane(o.rows_lo, k));
    const uint32_t lv = __builtin_amdgcn_readlane(o.left_vec, k);
    const int left = (int)(lv & 0xffffu);
    const bool vec = (lv >> 16) != 0;
    const int p = lane & 15;
    float* y = reinterpret_cast<float*>(yu);
#pragma unroll 1
    for (int i = 0; i < 4; ++i) {
        const int n = 4 * i + (lane >> 4);
        if (n < o.M) {
            const v4f v = *reinterpret_cast<const v4f*>(slot + (((p >> 2) * o.M + n) * 4 + (p & 3)) * 16);
            float* dst = y + (int64_t)n * rows + 4 * p;
            if (vec && 4 * p + 3 < left) {
                typedef __attribute__((address_space(1))) v4f global_v4f;
                __builtin_nontemporal_store(v, (global_v4f*)dst);
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * p + e < left) store_global_f32(dst + e, v[e]);
            }
        }
    }
}

// After the wave's last unit: the held units go out in order, each through
// its LDS slot (the units parked in registers pass through a slot already
// written out). (Called from inside the pipeline loop, at the last unit:
// after the loop, the same code makes the compiler keep ~50 more registers
// live across the loop.)
template <int TILES, int PARK>
__device__ __forceinline__ void mf_seq_flush(int lane, const MfOut& o, const MfPark<TILES, PARK>& park) {
    if constexpr (mf_seq_holds<TILES>()) {
        const int in_lds = min(o.k, o.slots);
        const int n = lane & 15, kg = lane >> 4;
#pragma unroll 1
        for (int k = 0; k < in_lds; ++k) mf_seq_store_slot<TILES>(o, k, o.lds + k * o.slot_bytes, lane);
#pragma unroll
        for (int i = 0; i < PARK; ++i)
            if (o.slots + i < o.k) {
                unsigned char* slot = o.lds + i * o.slot_bytes;  // slot i is written out: slots = 80 / M >= 5 > PARK
                if (n < o.M)
#pragma unroll
                    for (int t = 0; t < TILES; ++t)
                        *reinterpret_cast<v4f*>(slot + ((t * o.M + n) * 4 + kg) * 16) = park.acc[i][t];
                mf_seq_store_slot<TILES>(o, o.slots + i, slot, lane);
            }
    }
}

// One window of the pipeline: issue the loads of window `nxt` (computing its
// unit's addressing when it starts a unit), then the matrix work of window
// `cur`, then, at the end of cur's unit, hand its outputs on; after the wave's
// last unit (nothing follows cur), write out what LDS holds.
template <int KIND, int TILES, int XR, int PARK>
__device__ __forceinline__ void mf_seq_stage(const MfPos& nxt, MfUnit<TILES, XR>& un, MfWindow<KIND, TILES, XR>& into,
                                             const MfPos& cur, const MfWindow<KIND, TILES, XR>& have, bool last,
                                             int lane, v4f* acc, MfOut& out, MfPark<TILES, PARK>& park) {
    if (nxt.win == 0 && nxt.more) mf_unit<KIND>(un, nxt.d, nxt.v, lane);
    mf_seq_issue(into, un, nxt.d.K, nxt.win, lane);
    __builtin_amdgcn_sched_barrier(0);  // keep the next window's loads ahead of this window's matrix work
    mf_seq_compute(have, cur.d.K, cur.win, lane, acc);
    __builtin_amdgcn_sched_barrier(0);
    if (cur.win + 1 == cur.d.nwin) {
        mf_seq_retire<TILES, PARK>(cur.d, cur.v, lane, acc, out, park);
#pragma unroll
        for (int t = 0; t < TILES; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        if (last) mf_seq_flush<TILES, PARK>(lane, out, park);
    }
}

// Two register sets in turn: the loads of the next window are issued before
// the matrix work of the current one. M is the panel rows of every linear of
// the list.
template <int KIND, int TILES, int XR>
__global__ __launch_bounds__(kSeqWaves * kLanes) void k_mfseq(const MfSeqLin* __restrict__ lin,
                                                               const int64_t* __restrict__ pre, int64_t total, int M) {
    using Win = MfWindow<KIND, TILES, XR>;
    using Unit = MfUnit<TILES, XR>;
    extern __shared__ __attribute__((aligned(16))) unsigned char mf_lds[];
    const int lane = threadIdx.x % kLanes;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int64_t W = (int64_t)gridDim.x * kSeqWaves;
    MfPos p0;
    p0.u = (int64_t)xcd_contiguous_block() * kSeqWaves + wave;
    if (p0.u >= total) return;
    MfOut out;
    out.lds = mf_lds + wave * kMfSeqWaveLds;
    out.M = M;
    out.slot_bytes = TILES * M * 64;
    out.slots = mf_seq_holds<TILES>() && M >= kMfSeqHoldMinM ? kMfSeqWaveLds / out.slot_bytes : 0;
    out.k = 0;
    out.y_lo = out.y_hi = out.rows_lo = out.rows_hi = out.left_vec = 0;
    p0.win = 0;
    p0.j = 0;
    p0.more = true;
    while (p0.u >= pre[p0.j + 1]) ++p0.j;
    p0.d = lin[p0.j];
    p0.v = p0.u - pre[p0.j];
    Unit ua, ub;
    mf_unit<KIND>(ua, p0.d, p0.v, lane);
    v4f acc[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) acc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    // Registers for two more held units where they are free: the FP8 arm
    // where outputs are held. The bf16 arm's larger windows leave no room.
    constexpr int PARK = (KIND == 0 && mf_seq_holds<TILES>()) ? 2 : 0;
    MfPark<TILES, PARK> park;
    if constexpr (TILES == 4) {
        // Two register sets in turn: the loads of the next window are issued
        // before the matrix work of the current one.
        Win a, b;
        mf_seq_issue(a, ua, p0.d.K, p0.win, lane);
        for (;;) {
            const MfPos p1 = mf_next(p0, lin, pre, W, total);
            ub = ua;
            mf_seq_stage(p1, ub, b, p0, a, !p1.more, lane, acc, out, park);
            if (!p1.more) break;
            p0 = mf_next(p1, lin, pre, W, total);
            ua = ub;
            mf_seq_stage(p0, ua, a, p1, b, !p0.more, lane, acc, out, park);
            if (!p0.more) break;
        }
    } else {
        // Two-tile units hold half the bytes per window and leave registers
        // free: three sets in turn, the loads of the next two windows in
        // flight while a window's matrix work runs. `ua` follows the windows
        // as they are issued.
        Win a, b, c;
        mf_seq_issue(a, ua, p0.d.K, p0.win, lane);
        MfPos p1 = mf_next(p0, lin, pre, W, total);
        if (p1.win == 0 && p1.more) mf_unit<KIND>(ua, p1.d, p1.v, lane);
        mf_seq_issue(b, ua, p1.d.K, p1.win, lane);
        for (;;) {
            const MfPos p2 = mf_next(p1, lin, pre, W, total);
            mf_seq_stage(p2, ua, c, p0, a, !p1.more, lane, acc, out, park);
            if (!p1.more) break;
            const MfPos p3 = mf_next(p2, lin, pre, W, total);
            mf_seq_stage(p3, ua, a, p1, b, !p2.more, lane, acc, out, park);
            if (!p2.more) break;
            const MfPos p4 = mf_next(p3, lin, pre, W, total);
            mf_seq_stage(p4, ua, b, p2, c, !p3.more, lane, acc, out, park);
            if (!p3.more) break;
            p0 = p3;
            p1 = p4;
        }
    }
}

template <int KIND>
int mf_seq_launch(const fp8blk_sequence* seq, int arm, hipStream_t s) {
    if (!seq || !seq->plan || seq->arm != arm || seq->n < 1 || seq->M < 1 || seq->M > FP8BLK_MAX_M ||
        seq->units_dense < 1 || seq->grid_dense < 1)
        return FP8BLK_ERR_ARG;
    const MfSeqLin* lin = static_cast<const MfSeqLin*>(seq->plan);
    const int64_t* pre =
        reinterpret_cast<const int64_t*>(static_cast<const unsigned char*>(seq->plan) + (size_t)seq->n * sizeof(MfSeqLin));
    const dim3 nb((unsigned)seq->grid_dense), nt(kSeqWaves * kLanes);
    const int M = seq->M;
    // Where no outputs are held, the workgroup reserves only enough LDS to cap
    // a compute unit at the plan's workgroups (the units are dealt to the
    // waves in a fixed rotation, which assumes they progress at one rate).
    const int per_cu = mf_seq_blocks_per_cu(KIND == 0, M);
    const int lds = per_cu == kMfSeqBlocksPerCU ? kMfSeqLdsBytes : lds_cap_bytes(per_cu);
    (void)hipGetLastError();
    if (M >= 8)
        k_mfseq<KIND, mf_seq_tiles(8), 4><<<nb, nt, lds, s>>>(lin, pre, seq->units_dense, M);
    else if (M > 2)
        k_mfseq<KIND, mf_seq_tiles(3), 4><<<nb, nt, lds, s>>>(lin, pre, seq->units_dense, M);
    else if (M == 2)
        k_mfseq<KIND, mf_seq_tiles(2), 2><<<nb, nt, lds, s>>>(lin, pre, seq->units_dense, M);
    else
        k_mfseq<KIND, mf_seq_tiles(1), 1><<<nb, nt, lds, s>>>(lin, pre, seq->units_dense, M);
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

namespace fp8blk {
int64_t mf_sequence_plan(unsigned char* host, bool fp8, const fp8blk_seq_linear* linears, int n) {
    MfSeqLin* d = reinterpret_cast<MfSeqLin*>(host);
    int64_t* pre = reinterpret_cast<int64_t*>(host + (size_t)n * sizeof(MfSeqLin));
    pre[0] = 0;
    for (int j = 0; j < n; ++j) {
        const fp8blk_seq_linear& l = linears[j];
        MfSeqLin& s = d[j];
        s.w = l.w;
        s.grid = fp8 ? l.scales_f32 : nullptr;
        s.x = l.x_bf16;
        s.y = l.y;
        s.rows = l.rows;
        s.K = (int32_t)l.cols;
        s.M = (int32_t)l.M;
        s.GC = (int32_t)ceil_div(l.cols, kBlock);
        s.nwin = s.GC;
        s.vec_store = (l.rows % 4 == 0 && aligned(l.y, 16)) ? 1 : 0;
        s.pad = 0;
        pre[j + 1] = pre[j] + ceil_div(l.rows, (int64_t)kTile * mf_seq_tiles((int)l.M));
    }
    return pre[n];
}
}  // namespace fp8blk

extern "C" int fp8blk_gemv_mfma_sequence(const fp8blk_sequence* seq, fp8blk_stream_t stream) {
    return mf_seq_launch<0>(seq, FP8BLK_ARM_FP8_MFMA, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int bf16_gemv_twin_mfma_sequence(const fp8blk_sequence* seq, fp8blk_stream_t stream) {
    return mf_seq_launch<1>(seq, FP8BLK_ARM_BF16_MFMA, reinterpret_cast<hipStream_t>(stream));
}
