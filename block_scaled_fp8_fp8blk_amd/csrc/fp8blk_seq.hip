// Sequence launch: many independent M = 1 linears streamed by one persistent
// kernel, each output computed exactly as a call of its own.
//
// "Struct Dsv4Gpu" page, field dense_fp8: a decode step reads its dense
// linears as stored, and their weights are most of the step's bytes. Small
// linears launched one at a time leave HBM idle while each launch ramps up
// and drains; here the whole list is one stream of steps that every wave
// walks in list order, so the loads of the next linear are in flight while
// the current one finishes, and there is one launch for the list (two when
// some linears have ragged rows or cols: those units take a second launch of
// the same kernel with clamped addresses).
//
// Work: a step is S chunk slots per lane (S = 16 on the FP8 arm, 8 on the
// twin; 16 KB of weights per wave either way). Linear j is cut into units of
// R = S >> tl consecutive rows, tl = log2 of the segments of a row that one
// step covers: S/4 rows x 4 segments (T >= 3), S/2 rows x 2 segments (T = 2),
// S rows x 1 segment (T = 1). A unit of a linear with T <= 4 segments is one
// step; with T > 4 it is ceil(T / 4) steps of 4 segments of its rows, walked
// in segment order. Units are numbered across the list in order, and wave w
// of the W waves in the grid takes units w, w + W, w + 2W, ...: the waves
// move through the list together. Each wave issues the next step's loads
// (codes, x chunks, block scales) phase by phase, each phase just before it
// computes the same phase of the current step.
//
// Arithmetic per output (the order the library header documents):
//   lane partial = FMA chain over the chunk's 16 columns from +0.0;
//   segment sum  = tree64 over the lanes (tree64xV below);
//   y = P[0] + P[1] + ... + P[T-1] left to right (a running sum carried
//       across the steps of a unit when T > 4).
// This is the arithmetic of fp8blk_gemv / bf16_gemv_twin at M = 1, so each y
// is bitwise the same as from a call of its own.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

constexpr int kSeqThreads = kSeqWaves * kLanes;
constexpr int kSeqBlocksPerCU = 2;            // workgroups per compute unit
// Each workgroup reserves this much LDS (it uses none), so that no compute
// unit can hold more than kSeqBlocksPerCU of them (160 KB of LDS per CU): the
// units are dealt to the waves in a fixed rotation, which assumes every wave
// progresses at the same rate, and a CU holding one workgroup more than
// another would finish last.
constexpr int kSeqLdsBytes = lds_cap_bytes(kSeqBlocksPerCU);

// Device descriptor of one linear: 64 bytes of 32- and 64-bit fields, one
// scalar load.
struct alignas(64) SeqLin {
    const void* w;        // codes [rows, K] (FP8) or bf16 slab [rows, K] (twin)
    const float* grid;    // f32 block scales [ceil(rows/128), ceil(K/128)] (FP8 arm)
    const uint16_t* x;    // bf16 [K]
    float* y;             // f32 [rows]
    int64_t rows;
    int64_t dense_units;  // units on the dense path: 0 .. dense_units - 1
    int32_t K;            // cols
    int32_t T;            // segments, ceil(K / 1024)
    int32_t tl;           // log2 of segments of a row per step: 2 (T >= 3), 1 (T = 2), 0 (T = 1)
    int32_t Q;            // steps per unit: ceil(T / 4)
};
static_assert(sizeof(SeqLin) == 64, "one scalar load per descriptor");

static_assert(sizeof(SeqLin) == kSeqDescBytes, "descriptor size of the plan");

enum Kind { kFp8 = 0, kBf16 = 1 };

// Chunk slots per lane per step: 16 for the FP8 arm (16 KB of codes per wave
// step), 8 for the bf16 twin (the same bytes per step at 2 bytes a weight).
// Measured on the whole-step sweep: 8 FP8 slots run ~4% slower; 16 bf16 slots
// need more registers than two waves per SIMD allow.
constexpr int seq_slots(int kind) { return kind == kFp8 ? 16 : 8; }

// A step: chunk slot s (0 .. S-1) holds row r0 + (s >> tl) and segment
// 4k + (s & (tpw - 1)); x position p (0..3) holds the x chunk of segment
// 4k + (p & (tpw - 1)). Slot s then always meets the x chunk of position s & 3,
// whatever tl is. Scale position p holds, in lane l, the block scale of column
// block 8 (4k + (p & (tpw - 1))) + l / 8 of the unit's row block (R <= 16 rows
// that start at a multiple of R never cross a 128-row block): the scale of the
// lane's chunk in the segments of position p.
template <int KIND>
struct SeqRaw;

template <>
struct SeqRaw<kFp8> {
    uint4 c[seq_slots(kFp8)];
    uint4 x[4][2];
    float s[4];
};

template <>
struct SeqRaw<kBf16> {
    uint4 c[seq_slots(kBf16)][2];
    uint4 x[4][2];
};

constexpr int el_bytes(int kind) { return kind == kFp8 ? 1 : 2; }
__device__ __forceinline__ int grid_cols(const SeqLin& L) { return (L.K + kBlock - 1) / kBlock; }

// The loads of a step come in four phases, one per x position p: the code
// chunks of slots p, p + 4, p + 8, ... (segment p of every row of the step),
// the x chunk of position p and, on the FP8 arm, the block scales of position
// p. The arithmetic takes the same phases in the same order, so a wave can
// issue the next step's phase p just before it computes this step's phase p
// and keep one step of loads in flight at an even rate.
//
// The dense path: a unit whose R rows all exist, of a linear with K = 1024,
// K = 2048 or K a multiple of 4096. The step's slots then lie at
//   unit base + (s >> 2) * H + (s & 3) * 1024 weights,
// H = K for tl = 2 (the unit's next row) and H = 4096 otherwise (the slots
// continue one contiguous run of rows), and every chunk and scale index is
// in range with no clamping: each load is a wave-uniform base plus the lane's
// fixed offset.
template <int KIND>
__device__ __forceinline__ void load_dense(const SeqLin& L, int64_t v, int k, int lane, int p, SeqRaw<KIND>& raw) {
    constexpr int E = el_bytes(KIND);
    constexpr int S = seq_slots(KIND);
    const int tl = L.tl, tm = (1 << tl) - 1;
    const int64_t r0 = v * (S >> tl);
    const char* b0 = static_cast<const char*>(L.w) + (r0 * L.K + (int64_t)k * 4 * kSegCols) * E;
    const int64_t H = (tl == 2 ? L.K : 4 * kSegCols) * E;
    // FP8: lane l reads its chunk's 16 bytes, one 1 KB run per instruction.
    // bf16: a chunk is 32 bytes, and two loads of lane l's own 16-byte halves
    // would each touch every line of the segment's 2 KB half-used. Instead
    // load 0 reads the first KB and load 1 the second, lane m taking 16-byte
    // piece 2m (m < 32) or 2(m - 32) + 1 (m >= 32) of it; swap_lane_halves in
    // compute_phase then hands lane l pieces 2l and 2l + 1, its chunk. Measured on the whole-step sweep: 1.14 -> 0.92 ms per step
    // with contiguous loads.
    const uint32_t lo = KIND == kFp8 ? (uint32_t)lane * kChunk : 16u * (lane < 32 ? 2 * lane : 2 * lane - 63);
#pragma unroll
    for (int s = p; s < S; s += 4) {
        const char* a = b0 + (s >> 2) * H + p * kSegCols * E + lo;
        if constexpr (KIND == kFp8) {
            raw.c[s] = load_stream16(a);
        } else {
            raw.c[s][0] = load_stream16(a);
            raw.c[s][1] = load_stream16(a + kSegCols);
        }
    }
    const char* xp = reinterpret_cast<const char*>(L.x) + ((int64_t)k * 4 + (p & tm)) * kSegCols * 2 + (uint32_t)lane * 32;
    raw.x[p][0] = load_global16(xp);
    raw.x[p][1] = load_global16(xp + 16);
    if constexpr (KIND == kFp8)
        raw.s[p] = load_global_f32(L.grid + (r0 >> 7) * grid_cols(L) + 32 * k + 8 * (p & tm) + (lane >> 3));
}

// The general path: any K (a multiple of 16) and a last unit with fewer than
// R rows. Rows past the end re-read the last row and chunks past the last
// column re-read the last chunk; both are discarded by compute_phase.
template <int KIND>
__device__ __forceinline__ void load_general(const SeqLin& L, int64_t v, int k, int lane, int p, SeqRaw<KIND>& raw) {
    constexpr int E = el_bytes(KIND);
    constexpr int S = seq_slots(KIND);
    const int tl = L.tl, tm = (1 << tl) - 1;
    const int64_t r0 = v * (S >> tl);
    const char* wb = static_cast<const char*>(L.w) + (int64_t)k * 4 * kSegCols * E;
    const int qmax = L.K / kChunk - 1 - 4 * k * kLanes;  // last chunk, relative to the step
#pragma unroll
    for (int s = p; s < S; s += 4) {
        const int64_t row = min(r0 + (s >> tl), L.rows - 1);
        const uint32_t off = (uint32_t)min((s & tm) * kLanes + lane, qmax) * (kChunk * E);
        const char* a = wb + row * L.K * E + off;
        if constexpr (KIND == kFp8) {
            raw.c[s] = load_stream16(a);
        } else {
            raw.c[s][0] = load_stream16(a);
            raw.c[s][1] = load_stream16(a + 16);
        }
    }
    const char* xp = reinterpret_cast<const char*>(L.x) + (int64_t)k * 4 * kSegCols * 2 +
                     (uint32_t)min((p & tm) * kLanes + lane, qmax) * (kChunk * 2);
    raw.x[p][0] = load_global16(xp);
    raw.x[p][1] = load_global16(xp + 16);
    if constexpr (KIND == kFp8) {
        const int gc = grid_cols(L);
        raw.s[p] = load_global_f32(L.grid + (min(r0, L.rows - 1) >> 7) * gc +
                                   min(32 * k + 8 * (p & tm) + (lane >> 3), gc - 1));
    }
}

template <int KIND, bool DENSE>
__device__ __forceinline__ void load_phase(const SeqLin& L, int64_t v, int k, int lane, int p, SeqRaw<KIND>& raw) {
    if constexpr (DENSE)
        load_dense<KIND>(L, v, k, lane, p, raw);
    else
        load_general<KIND>(L, v, k, lane, p, raw);
}

template <int KIND, bool DENSE>
__device__ __forceinline__ void load_step(const SeqLin& L, int64_t v, int k, int lane, SeqRaw<KIND>& raw) {
#pragma unroll
    for (int p = 0; p < 4; ++p) load_phase<KIND, DENSE>(L, v, k, lane, p, raw);
}

// Phase p of the arithmetic of step k: the lane partials of slots p, p + 4,
// ... (one FMA chain over each chunk's 16 columns, from +0.0), into part.
template <int KIND, bool DENSE>
__device__ __forceinline__ void compute_phase(const SeqLin& L, int k, int lane, int p, const SeqRaw<KIND>& raw,
                                              float (&part)[seq_slots(KIND)]) {
    constexpr int S = seq_slots(KIND);
    const int tl = L.tl;
    const int tpw = 1 << tl;
    float xf[kChunk];
    widen8_bf16(raw.x[p][0], xf);
    widen8_bf16(raw.x[p][1], xf + 8);
#pragma unroll
    for (int s = p; s < S; s += 4) {
        float w[kChunk];
        if constexpr (KIND == kFp8) {
            decode16_fp8_scaled(raw.c[s], raw.s[p], w);
        } else if constexpr (DENSE) {
            // the dense path's pieces (load_dense) -> the lane's own chunk,
            // lower half first
            uint4 lo = raw.c[s][0], hi = raw.c[s][1];
            swap_lane_halves(lo, hi);
            widen8_bf16(lo, w);
            widen8_bf16(hi, w + 8);
        } else {
            widen8_bf16(raw.c[s][0], w);
            widen8_bf16(raw.c[s][1], w + 8);
        }
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kChunk; ++j) acc = __builtin_fmaf(w[j], xf[j], acc);
        if constexpr (DENSE) {
            part[s] = acc;  // every chunk of a dense step exists
        } else {
            const int us = s & (tpw - 1);
            const int nseg = min(tpw, L.T - 4 * k);  // live segments of a row in this step
            const bool live = us < nseg && us * kLanes + lane <= L.K / kChunk - 1 - 4 * k * kLanes;
            part[s] = live ? acc : 0.0f;
        }
    }
}

// The end of step k of unit v: segment sums (tree64xV) and the row sums in
// segment order; yacc carries the running sums of the rows of a unit across
// its steps (tl = 2). Stores after the unit's last step.
template <int KIND, bool DENSE>
__device__ __forceinline__ void finish_step(const SeqLin& L, int64_t v, int k, int lane,
                                            float (&part)[seq_slots(KIND)], float (&yacc)[seq_slots(KIND) / 4]) {
    constexpr int S = seq_slots(KIND), NR = S / 4;
    const int tl = L.tl;
    const int nseg = min(1 << tl, L.T - 4 * k);
    float red[NR];
    tree64xV<S>(part, red);
    // segment sum of slot s, uniform across the wave
    float P[S];
#pragma unroll
    for (int s = 0; s < S; ++s) P[s] = lane_value(red[s >> 2], 16 * kRowOf4[s & 3]);

    const int64_t r0 = v * (S >> tl);
    float out;
    if (tl == 2) {  // NR rows, four segments of each
        float y[NR];
#pragma unroll
        for (int h = 0; h < NR; ++h) {
            y[h] = (k == 0) ? P[4 * h] : yacc[h] + P[4 * h];
#pragma unroll
            for (int us = 1; us < 4; ++us)
                if (DENSE || us < nseg) y[h] = y[h] + P[4 * h + us];
            yacc[h] = y[h];
        }
        if (k + 1 < L.Q) return;
        out = y[NR - 1];
#pragma unroll
        for (int h = NR - 2; h >= 0; --h)
            if (lane == h) out = y[h];
    } else if (tl == 1) {  // 2 * NR rows, two segments each
        out = P[S - 2] + P[S - 1];
#pragma unroll
        for (int i = S / 2 - 2; i >= 0; --i)
            if (lane == i) out = P[2 * i] + P[2 * i + 1];
    } else {  // 4 * NR rows, one segment each
        out = P[S - 1];
#pragma unroll
        for (int i = S - 2; i >= 0; --i)
            if (lane == i) out = P[i];
    }
    const int R = S >> tl;
    if (lane < R && r0 + lane < L.rows) store_global_f32(L.y + r0 + lane, out);
}

// Where a wave is in the list: unit u (global numbering within the path),
// v = the unit's index within its linear, step k of it, its linear j and that
// linear's descriptor.
struct SeqPos {
    int64_t u, v;
    int k, j;
    bool more;  // false: past the wave's last step (the position is the last step again)
    SeqLin L;
};

// The step after p: the next step of the unit, else the wave's next unit.
// Past the wave's last step the last step is repeated (its loads are issued
// and discarded), so every stage of the loop below issues the same loads.
// `first` maps a path-local unit index to the unit index within the linear:
// 0 on the dense path, the linear's dense_units on the general one.
template <bool DENSE>
__device__ __forceinline__ SeqPos next_pos(const SeqPos& p, const SeqLin* lin, const int64_t* pre, int64_t W,
                                           int64_t total) {
    SeqPos n = p;
    if (!p.more) return n;
    if (p.k + 1 < p.L.Q) {
        n.k = p.k + 1;
    } else if (p.u + W < total) {
        n.u = p.u + W;
        n.v = p.v + W;
        n.k = 0;
        if (n.u >= pre[n.j + 1]) {
            do ++n.j;
            while (n.u >= pre[n.j + 1]);
            n.L = lin[n.j];
            n.v = n.u - pre[n.j] + (DENSE ? 0 : n.L.dense_units);
        }
    } else {
        n.more = false;
    }
    return n;
}

// Issue the loads of step `nxt` phase by phase, each just before the same
// phase of the arithmetic of step `cur`; then finish `cur`.
template <int KIND, bool DENSE>
__device__ __forceinline__ void stage(const SeqPos& nxt, SeqRaw<KIND>& into, const SeqPos& cur,
                                      const SeqRaw<KIND>& have, int lane, float (&yacc)[seq_slots(KIND) / 4]) {
    float part[seq_slots(KIND)];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        load_phase<KIND, DENSE>(nxt.L, nxt.v, nxt.k, lane, p, into);
        __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the phase's arithmetic
        compute_phase<KIND, DENSE>(cur.L, cur.k, lane, p, have, part);
        __builtin_amdgcn_sched_barrier(0);
    }
    finish_step<KIND, DENSE>(cur.L, cur.v, cur.k, lane, part, yacc);
}

// One path (dense or general) of a sequence: `total` units, linear j owning
// path units [pre[j], pre[j + 1]). Two register sets in turn: the loads of
// the next step are issued before the arithmetic of the current one, and no
// register copy makes the wave wait for loads it does not need yet.
template <int KIND, bool DENSE>
__global__ __launch_bounds__(kSeqThreads) void k_seq(const SeqLin* __restrict__ lin, const int64_t* __restrict__ pre,
                                                     int64_t total) {
    const int lane = threadIdx.x % kLanes;
    const int64_t W = (int64_t)gridDim.x * kSeqWaves;
    SeqPos p0;
    p0.u = (int64_t)xcd_contiguous_block() * kSeqWaves + __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    if (p0.u >= total) return;
    p0.k = 0;
    p0.j = 0;
    p0.more = true;
    while (p0.u >= pre[p0.j + 1]) ++p0.j;
    p0.L = lin[p0.j];
    p0.v = p0.u - pre[p0.j] + (DENSE ? 0 : p0.L.dense_units);
    float yacc[seq_slots(KIND) / 4] = {};
    SeqRaw<KIND> a, b;
    load_step<KIND, DENSE>(p0.L, p0.v, p0.k, lane, a);
    for (;;) {
        const SeqPos p1 = next_pos<DENSE>(p0, lin, pre, W, total);
        stage<KIND, DENSE>(p1, b, p0, a, lane, yacc);
        if (!p1.more) break;
        p0 = next_pos<DENSE>(p1, lin, pre, W, total);
        stage<KIND, DENSE>(p0, a, p1, b, lane, yacc);
        if (!p0.more) break;
    }
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" size_t fp8blk_sequence_bytes(int n) {
    if (n < 1 || n > FP8BLK_MAX_SEQ) return 0;
    return plan_bytes(n);
}

extern "C" int fp8blk_sequence_init(fp8blk_sequence* seq, int arm, const fp8blk_seq_linear* linears, int n,
                                    void* ws, size_t ws_bytes, fp8blk_stream_t stream) {
    if (!seq || !linears || n < 1 || n > FP8BLK_MAX_SEQ || arm < FP8BLK_ARM_FP8 || arm > FP8BLK_ARM_BF16_MFMA)
        return FP8BLK_ERR_ARG;
    if (!ws || !aligned(ws, 64) || ws_bytes < plan_bytes(n)) return FP8BLK_ERR_WORKSPACE;
    const bool fp8 = arm == FP8BLK_ARM_FP8 || arm == FP8BLK_ARM_FP8_MFMA;
    const bool mfma = arm == FP8BLK_ARM_FP8_MFMA || arm == FP8BLK_ARM_BF16_MFMA;
    const int64_t M = linears[0].M;
    for (int j = 0; j < n; ++j) {
        const fp8blk_seq_linear& l = linears[j];
        if (!l.w || !l.x_bf16 || !l.y || !shape_ok(l.rows, l.cols) || !aligned(l.w, 16) || !aligned(l.x_bf16, 16) ||
            !aligned(l.y, 4) || l.M != M || M < 1 || M > (mfma ? FP8BLK_MAX_M : 1))
            return FP8BLK_ERR_ARG;
        if (fp8 && (!l.scales_f32 || !aligned(l.scales_f32, 4))) return FP8BLK_ERR_ARG;
    }
    std::vector<unsigned char> host(plan_bytes(n));
    int64_t units_first = 0, units_second = 0;
    if (mfma) {
        units_first = mf_sequence_plan(host.data(), fp8, linears, n);
    } else {
        SeqLin* d = reinterpret_cast<SeqLin*>(host.data());
        int64_t* pre_d = reinterpret_cast<int64_t*>(host.data() + (size_t)n * sizeof(SeqLin));
        int64_t* pre_g = pre_d + (n + 1);
        pre_d[0] = pre_g[0] = 0;
        for (int j = 0; j < n; ++j) {
            const fp8blk_seq_linear& l = linears[j];
            SeqLin& s = d[j];
            s.w = l.w;
            s.grid = fp8 ? l.scales_f32 : nullptr;
            s.x = l.x_bf16;
            s.y = l.y;
            s.rows = l.rows;
            s.K = (int32_t)l.cols;
            s.T = (int32_t)ceil_div(l.cols, kSegCols);
            s.tl = s.T >= 3 ? 2 : s.T == 2 ? 1 : 0;
            s.Q = (int32_t)ceil_div(s.T, 4);
            // Dense: every chunk slot of a step is a whole chunk of the row it
            // names (K = 1024, 2048 or a multiple of 4096) and the unit has all
            // its R rows; a last unit with fewer rows, and every unit of another
            // K, take the general path.
            const int64_t R = (fp8 ? seq_slots(kFp8) : seq_slots(kBf16)) >> s.tl;
            const bool dense = l.cols == kSegCols || l.cols == 2 * kSegCols || l.cols % (4 * kSegCols) == 0;
            s.dense_units = dense ? l.rows / R : 0;
            pre_d[j + 1] = pre_d[j] + s.dense_units;
            pre_g[j + 1] = pre_g[j] + (ceil_div(l.rows, R) - s.dense_units);
        }
        units_first = pre_d[n];
        units_second = pre_g[n];
    }
    const int cus = device_cus();
    if (cus < 1) return FP8BLK_ERR_HIP;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, st) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FP8BLK_ERR_HIP;
    const int64_t waves = (int64_t)cus * (mfma ? mf_seq_blocks_per_cu(fp8, M) : kSeqBlocksPerCU) * kSeqWaves;
    seq->plan = ws;
    seq->units_dense = units_first;
    seq->units_general = units_second;
    seq->n = n;
    seq->arm = arm;
    seq->grid_dense = (int32_t)ceil_div(std::min<int64_t>(waves, units_first), kSeqWaves);
    seq->grid_general = (int32_t)ceil_div(std::min<int64_t>(waves, units_second), kSeqWaves);
    seq->M = (int32_t)M;
    seq->reserved = 0;
    return FP8BLK_OK;
}

namespace {
template <int KIND>
int launch_seq(const fp8blk_sequence* seq, int arm, fp8blk_stream_t stream) {
    if (!seq || !seq->plan || seq->arm != arm || seq->n < 1 || seq->M != 1 || seq->units_dense < 0 || seq->units_general < 0 ||
        seq->units_dense + seq->units_general < 1 || (seq->units_dense > 0 && seq->grid_dense < 1) ||
        (seq->units_general > 0 && seq->grid_general < 1))
        return FP8BLK_ERR_ARG;
    const SeqLin* lin = static_cast<const SeqLin*>(seq->plan);
    const int64_t* pre_d = reinterpret_cast<const int64_t*>(static_cast<const unsigned char*>(seq->plan) +
                                                            (size_t)seq->n * sizeof(SeqLin));
    const int64_t* pre_g = pre_d + (seq->n + 1);
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (seq->units_dense > 0)
        k_seq<KIND, true><<<dim3((unsigned)seq->grid_dense), dim3(kSeqThreads), kSeqLdsBytes, st>>>(lin, pre_d,
                                                                                                 seq->units_dense);
    if (seq->units_general > 0)
        k_seq<KIND, false><<<dim3((unsigned)seq->grid_general), dim3(kSeqThreads), kSeqLdsBytes, st>>>(
            lin, pre_g, seq->units_general);
    return launch_status();
}
}  // namespace

extern "C" int fp8blk_gemv_sequence(const fp8blk_sequence* seq, fp8blk_stream_t stream) {
    return launch_seq<kFp8>(seq, FP8BLK_ARM_FP8, stream);
}

extern "C" int bf16_gemv_twin_sequence(const fp8blk_sequence* seq, fp8blk_stream_t stream) {
    return launch_seq<kBf16>(seq, FP8BLK_ARM_BF16, stream);
}
