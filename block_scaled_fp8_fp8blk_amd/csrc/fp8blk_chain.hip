// Chained launch: a dependent list of FP8-blk GEMV groups in one persistent,
// cooperative launch.
//
// The pages' device decode path runs one launch per projection ("Module
// dsv4_gpu" page, DecodePath), and each projection reads what the one before
// it wrote. On MI355X every launch of a 4-21 MB linear pays a ramp and a drain
// of ~2.5 us around ~2 us of streaming (a dependent step of 173 launches runs
// at ~42% of HBM peak). Here one launch runs the whole list: every group's
// weights do not depend on the activations, so each wave issues the loads of
// its next units while the group before is still being finished elsewhere,
// and only the (small) activation hand-off waits.
//
// Arithmetic: every output follows the documented order of fp8blk_gemv (lane
// chunks of 16 columns by a fused multiply-add chain from +0.0, a pairwise tree
// over the 64 lanes of a 1024-column segment, segments added left to right),
// so each y equals a fp8blk_gemv call on the same input bit for bit. The input
// of a group that reads an earlier linear's output is x = bf16(c * y) (the
// f32 product, rounded to nearest even): a per-group scale standing in for the
// elementwise work an engine does between projections.
//
// Hand-off: a linear whose output feeds a later group also writes each output
// as one 8-byte word (f32 bits, launch epoch) with a device-coherent store.
// In every workgroup one polling wave reads a group's input words (device-
// coherent loads, past the XCD's L2) until every word carries this launch's
// epoch, converts them into the group's bf16 input in LDS, and meets the
// compute waves at a barrier. The words validate themselves, so no counter,
// fence or reset is needed between groups; the epoch (a counter in the
// workspace, bumped by the last workgroup to finish) tells one launch's words
// from the previous one's. The compute waves never wait on memory for the
// hand-off (their weight loads stay in flight across it), and the polling
// wave's loads never queue behind weight loads.
//
// Every wait is bounded: a polling wave that has not seen its input after
// kChSpin polls records FP8BLK_ERR_TIMEOUT in the workspace; every polling
// wave that sees the record stops waiting, so the launch always runs to its
// end. The launch is cooperative (every workgroup resident at once), which
// the waits need.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

constexpr int kChWaves = 12;                 // waves per workgroup: kChWaves - 1 compute waves and one polling wave
constexpr int kChCompute = kChWaves - 1;
constexpr int kChPoller = kChWaves - 1;      // the polling wave's index
constexpr int kChSlots = 8;                  // 16-byte code chunks per lane per unit
constexpr int kChMaxCols = 4096;
constexpr int kChSpin = 1 << 21;             // polls before a wait gives up (seconds, far beyond any group)
constexpr int kChErrCheck = 64;              // polls between checks of the error record
// The polling wave reads a group's input no sooner than kChPollDelay ticks of
// the 100 MHz real-time counter after the barrier that released the group
// before it: the outputs it waits for take about that long to be computed
// and written (one unit of vector work and the write-through), and device-
// coherent polls issued earlier only slow every workgroup's weight loads.
// Measured on the 173-group decode chain (8-slot units): 1.15 ms per launch
// waiting 3.4 us, 1.10 ms waiting 2.0-2.7 us; with 16-slot units: 1.39 ms
// polling at once, 1.23-1.26 ms waiting 3.0-3.8 us, 1.41 ms waiting 5 us,
// and 1.46-1.57 ms waiting instead for the workgroup's own units to be
// stored.
constexpr uint64_t kChPollDelay = 240;
constexpr int kBufferWord3 = 0x00020000;     // buffer resource word 3: raw 32-bit data
constexpr int kCoherent = 16;                // cache policy of a device-coherent load (sc1)

// Control words at the start of the workspace, one per 64 bytes.
constexpr int kCtlEpoch = 0, kCtlDone = 16, kCtlErr = 32;
constexpr size_t kCtlBytes = 256;

// One work unit (8 chunk slots of one linear, 8 / T4 consecutive rows):
// everything its loads, arithmetic and stores need, precomputed on the host,
// so that the loop reads no descriptor (a scalar load would be waited for at
// every barrier).
struct alignas(16) ChRec {
    const uint8_t* w;    // codes of the unit's first row
    const float* grid;   // the unit's row of block scales
    float* y;            // output of the unit's first row
    int32_t ll;          // word index of that output among the linked outputs, -1: none
    int32_t left;        // rows of the unit that exist (<= 8 / T4)
    int32_t cols;        // 1024, 2048, 3072 or 4096
    int32_t group;
};
static_assert(sizeof(ChRec) == 48, "three 16-byte loads per record");

struct alignas(16) ChGroup {
    int32_t cols;
    int32_t src_ll;     // word index of the input's linked outputs; -1: the chain input x0
    float c;
    int32_t pad;
};
static_assert(sizeof(ChGroup) == 16, "one 16-byte load per group");

struct ChArgs {
    const ChRec* recs;
    const ChGroup* groups;
    uint64_t* ll;         // linked outputs (8-byte words)
    uint32_t* ctl;        // control words
    const uint16_t* x0;
    int64_t units;
    int32_t n_groups;
};

// Rows per unit: 8 chunk slots per lane, T4 segments per row (T4 = 1, 2 or 4;
// cols 3072 use four slots per row, the last one unused).
__host__ __device__ constexpr int seg_slots(int cols) { return cols <= 1024 ? 1 : cols <= 2048 ? 2 : 4; }

// The records of 64 consecutive units of a wave (lane l: its unit k0 + l),
// read lane by lane into scalar registers.
struct ChRecs {
    uint4 a, b, c;
    int64_t k0;
};

struct ChItem {
    const uint8_t* w;
    const float* grid;
    float* y;
    int32_t ll, left, cols, group;
    bool more;
};

__device__ __forceinline__ void ch_recs_load(ChRecs& R, const ChArgs& a, int64_t gw, int64_t W, int64_t k0, int lane) {
    const int64_t u = min(gw + (k0 + lane) * W, a.units - 1);
    const uint4* p = reinterpret_cast<const uint4*>(a.recs + u);
    R.a = load_global16(p);
    R.b = load_global16(p + 1);
    R.c = load_global16(p + 2);
    R.k0 = k0;
}

__device__ __forceinline__ uint64_t rl64(uint32_t lo, uint32_t hi, int l) {
    return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)hi, l) << 32) | (uint32_t)__builtin_amdgcn_readlane((int)lo, l);
}

// Item k of the wave (k < n_items; a k past the end repeats the last one with
// more = false, whose loads stay valid).
__device__ __forceinline__ ChItem ch_item(ChRecs& R, const ChArgs& a, int64_t gw, int64_t W, int64_t k, int64_t n_items,
                                          int lane) {
    ChItem it;
    it.more = k < n_items;
    const int64_t kk = it.more ? k : n_items > 0 ? n_items - 1 : 0;  // a wave with no unit reads record 0 of its list
    if (kk < R.k0 || kk >= R.k0 + kLanes) ch_recs_load(R, a, gw, W, kk - kk % kLanes, lane);
    const int l = (int)(kk - R.k0);
    it.w = reinterpret_cast<const uint8_t*>(rl64(R.a.x, R.a.y, l));
    it.grid = reinterpret_cast<const float*>(rl64(R.a.z, R.a.w, l));
    it.y = reinterpret_cast<float*>(rl64(R.b.x, R.b.y, l));
    it.ll = __builtin_amdgcn_readlane((int)R.b.z, l);
    it.left = __builtin_amdgcn_readlane((int)R.b.w, l);
    it.cols = __builtin_amdgcn_readlane((int)R.c.x, l);
    it.group = __builtin_amdgcn_readlane((int)R.c.y, l);
    return it;
}

struct ChRaw {
    uint4 c[kChSlots];
    float s;  // lane k: block scale k of the unit's row block (k < 8 * T4)
};

// The loads of one unit: slot s is row s / T4, segment s % T4; lane l takes
// chunk 64 t + l. Rows past the unit's last row and chunks past the last
// column re-read the last one (their results are not used).
template <int T4>
__device__ __forceinline__ void ch_issue(ChRaw& r, const ChItem& I, int lane) {
    const int last_q = I.cols / 16 - 1;
#pragma unroll
    for (int s = 0; s < kChSlots; ++s) {
        const int i = min(s / T4, I.left - 1), t = s % T4;
        const int q = min(64 * t + lane, last_q);
        r.c[s] = load_stream16(I.w + (int64_t)i * I.cols + 16 * q);
    }
    r.s = load_global_f32(I.grid + min(lane, I.cols / kBlock - 1));
}

__device__ __forceinline__ void ch_issue_any(ChRaw& r, const ChItem& I, int lane) {
    const int T4 = seg_slots(I.cols);
    if (T4 == 4)
        ch_issue<4>(r, I, lane);
    else if (T4 == 2)
        ch_issue<2>(r, I, lane);
    else
        ch_issue<1>(r, I, lane);
}

// One unit's outputs, from its loads and the group's bf16 input in LDS.
template <int T4>
__device__ __forceinline__ void ch_compute(const ChRaw& r, const ChItem& I, const uint4* xs, int lane, uint32_t epoch,
                                           uint64_t* ll) {
    constexpr int R = kChSlots / T4;
    const int T = I.cols / 1024;  // segments that exist (T <= T4)
    float v[kChSlots];
#pragma unroll
    for (int t = 0; t < T4; ++t) {
        const int q = 64 * t + lane;
        float xf[kChunk];
        const uint4 x0 = xs[2 * q], x1 = xs[2 * q + 1];
        widen8_bf16(x0, xf);
        widen8_bf16(x1, xf + 8);
        const float sc = __shfl(r.s, 8 * t + (lane >> 3));
#pragma unroll
        for (int i = 0; i < R; ++i) {
            float w[kChunk];
            decode16_fp8_scaled(r.c[i * T4 + t], sc, w);
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < kChunk; ++j) s = __builtin_fmaf(w[j], xf[j], s);
            v[i * T4 + t] = t < T ? s : 0.0f;
        }
    }
    float red[kChSlots / 4];
    tree64xV<kChSlots>(v, red);
    // Lane i < R gathers the segment sums of row i (value i T4 + t sits in
    // register (i T4 + t) / 4, lane row kRowOf4[(i T4 + t) % 4]) and adds them
    // left to right.
    float out = 0.0f;
#pragma unroll
    for (int t = 0; t < T4; ++t) {
        const int vi = min(lane, R - 1) * T4 + t;
        const int src = 16 * (((vi & 1) << 1) | ((vi >> 1) & 1));  // 16 kRowOf4[vi % 4]
        float p = 0.0f;
#pragma unroll
        for (int k = 0; k < kChSlots / 4; ++k) {
            const float sk = __shfl(red[k], src);
            if (vi / 4 == k) p = sk;
        }
        out = t == 0 ? p : t < T ? out + p : out;
    }
    if (lane < I.left) {
        store_global_f32(I.y + lane, out);
        if (I.ll >= 0) {
            const uint64_t word = ((uint64_t)epoch << 32) | as_u32(out);
            __hip_atomic_store(ll + I.ll + lane, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__device__ __forceinline__ void ch_compute_any(const ChRaw& r, const ChItem& I, const uint4* xs, int lane,
                                               uint32_t epoch, uint64_t* ll) {
    const int T4 = seg_slots(I.cols);
    if (T4 == 4)
        ch_compute<4>(r, I, xs, lane, epoch, ll);
    else if (T4 == 2)
        ch_compute<2>(r, I, xs, lane, epoch, ll);
    else
        ch_compute<1>(r, I, xs, lane, epoch, ll);
}

__device__ __forceinline__ uint32_t ld_coherent_u32(uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The polling wave's reads of one group's input words: NP 16-byte pieces
// (two words each) per lane, lane l taking pieces l + 64 k. It first waits on
// a sample (every eighth piece: one eighth of the device-coherent reads per
// poll, which all 256 workgroups repeat), then reads every piece until every
// word carries this launch's epoch, and writes the bf16 input into LDS.
template <int NP>
__device__ __forceinline__ void ch_poll_words(const ChArgs& a, int src_ll, float c, uint4* xs, int lane,
                                              uint32_t epoch) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(a.ll + src_ll, (short)0, NP * kLanes * 16, kBufferWord3);
    uint32_t* x32 = reinterpret_cast<uint32_t*>(xs);
    for (int it = 0; it < kChSpin; ++it) {
        bool ok = true;
#pragma unroll
        for (int k = 0; k < NP; k += 8) {
            const auto t = __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + kLanes * k) * 16, 0, kCoherent);
            ok = ok && t[1] == epoch && t[3] == epoch;
        }
        if (__all(ok)) break;
        if (it % kChErrCheck == kChErrCheck - 1 && __builtin_amdgcn_readfirstlane(ld_coherent_u32(a.ctl + kCtlErr)) != 0)
            break;
        __builtin_amdgcn_s_sleep(1);
    }
    for (int it = 0;; ++it) {
        // in halves of at most 16 pieces per lane (registers); each half's bf16
        // input goes to LDS as it is read, and counts only if every half carried
        // the epoch in the same pass
        bool ok = true;
#pragma unroll
        for (int h = 0; h < NP; h += 16) {
            uint4 v[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (h + k < NP) {
                    const auto t =
                        __builtin_amdgcn_raw_buffer_load_b128(rs, (lane + kLanes * (h + k)) * 16, 0, kCoherent);
                    v[k] = make_uint4(t[0], t[1], t[2], t[3]);
                }
#pragma unroll
            for (int k = 0; k < 16; ++k)
                if (h + k < NP) {
                    ok = ok && v[k].y == epoch && v[k].w == epoch;
                    x32[lane + kLanes * (h + k)] = bf16_of_scaled(c, v[k].x) | (bf16_of_scaled(c, v[k].z) << 16);
                }
        }
        bool stop = __all(ok);
        if (!stop && it >= kChSpin) {
            if (lane == 0) __hip_atomic_fetch_or(a.ctl + kCtlErr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            stop = true;
        }
        if (!stop && it % kChErrCheck == kChErrCheck - 1)
            stop = __builtin_amdgcn_readfirstlane(ld_coherent_u32(a.ctl + kCtlErr)) != 0;
        if (stop) return;
        __builtin_amdgcn_s_sleep(1);
    }
}

// The polling wave: group g's bf16 input into LDS slot xs. gd: lane l holds
// the descriptor of group g - g % 64 + l.
__device__ __forceinline__ void ch_poll(const ChArgs& a, int g, const uint4& gd, uint4* xs, int lane, uint32_t epoch) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    const int l = g % kLanes;
    const int cols = __builtin_amdgcn_readlane((int)gd.x, l);
    const int src_ll = __builtin_amdgcn_readlane((int)gd.y, l);
    const float c = as_f32((uint32_t)__builtin_amdgcn_readlane((int)gd.z, l));
    if (src_ll < 0) {
        const uint4* src = reinterpret_cast<const uint4*>(a.x0);
        for (int p = lane; p < cols / 8; p += kLanes) xs[p] = load_global16(src + p);
        return;
    }
    while (__builtin_amdgcn_s_memrealtime() - t0 < kChPollDelay) __builtin_amdgcn_s_sleep(8);
    switch (cols) {
        case 1024: ch_poll_words<8>(a, src_ll, c, xs, lane, epoch); break;
        case 2048: ch_poll_words<16>(a, src_ll, c, xs, lane, epoch); break;
        case 3072: ch_poll_words<24>(a, src_ll, c, xs, lane, epoch); break;
        default: ch_poll_words<32>(a, src_ll, c, xs, lane, epoch); break;
    }
}

__global__ __launch_bounds__(kChWaves * kLanes) void k_chain(const ChArgs a) {
    __shared__ uint4 xs[2][kChMaxCols * 2 / 16];
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
    const int lane = threadIdx.x % kLanes;
    const uint32_t epoch = ld_coherent_u32(a.ctl + kCtlEpoch) + 1u;

    if (wave == kChPoller) {
        uint4 gd = make_uint4(0, 0, 0, 0);
        for (int g = 0; g < a.n_groups; ++g) {
            if (g % kLanes == 0) gd = load_global16(a.groups + min(g + lane, a.n_groups - 1));
            ch_poll(a, g, gd, xs[g & 1], lane, epoch);
            __syncthreads();
        }
    } else {
        // compute wave gw of W takes units gw, gw + W, ...: its items k = 0, 1, ...
        const int64_t W = (int64_t)gridDim.x * kChCompute;
        const int64_t gw = (int64_t)blockIdx.x * kChCompute + wave;
        const int64_t n_items = gw < a.units ? (a.units - 1 - gw) / W + 1 : 0;
        ChRecs R;
        ch_recs_load(R, a, gw, W, 0, lane);
        int64_t k = 0;
        ChItem I0 = ch_item(R, a, gw, W, k, n_items, lane);
        ChItem I1 = ch_item(R, a, gw, W, k + 1, n_items, lane);
        ChRaw A, B;
        ch_issue_any(A, I0, lane);
        ch_issue_any(B, I1, lane);
        int gx = 0;  // barriers passed = groups whose input is in LDS
        // two register sets in turn: item k + 2 is loaded into a set as soon
        // as item k has been computed from it
        for (;;) {
            if (!I0.more) break;
            for (; gx <= I0.group; ++gx) __syncthreads();
            ch_compute_any(A, I0, xs[(gx - 1) & 1], lane, epoch, a.ll);
            I0 = ch_item(R, a, gw, W, k + 2, n_items, lane);
            ch_issue_any(A, I0, lane);
            if (!I1.more) break;
            for (; gx <= I1.group; ++gx) __syncthreads();
            ch_compute_any(B, I1, xs[(gx - 1) & 1], lane, epoch, a.ll);
            I1 = ch_item(R, a, gw, W, k + 3, n_items, lane);
            ch_issue_any(B, I1, lane);
            k += 2;
        }
        for (; gx < a.n_groups; ++gx) __syncthreads();
    }
    // The last workgroup to finish moves the epoch on for the next launch
    // (every workgroup read it at its start).
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t d = __hip_atomic_fetch_add(a.ctl + kCtlDone, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d + 1 == gridDim.x) {
            __hip_atomic_store(a.ctl + kCtlDone, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(a.ctl + kCtlEpoch, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Workspace layout: control words, group descriptors, one record per work
// unit (units numbered over the list in order), linked outputs (one 8-byte
// word per output row of every linear that feeds a later group).
struct ChLayout {
    size_t groups, recs, ll, total;
    int64_t units, ll_words;
};

size_t align64(size_t b) { return (b + 63) & ~(size_t)63; }

bool ch_valid(const fp8blk_linear* lins, int n_lins, const fp8blk_chain_group* groups, int n_groups) {
    if (!lins || !groups || n_lins < 1 || n_groups < 1 || n_lins > FP8BLK_MAX_CHAIN || n_groups > n_lins) return false;
    int next = 0;
    for (int g = 0; g < n_groups; ++g) {
        const fp8blk_chain_group& G = groups[g];
        if (G.first != next || G.n < 1 || G.first + G.n > n_lins) return false;
        if (G.cols != 1024 && G.cols != 2048 && G.cols != 3072 && G.cols != 4096) return false;
        if (G.src >= 0) {
            if (G.src >= G.first || lins[G.src].rows != G.cols) return false;
            if (!(G.c == G.c)) return false;
        } else if (G.src != -1) {
            return false;
        }
        for (int j = G.first; j < G.first + G.n; ++j) {
            const fp8blk_linear& L = lins[j];
            if (!L.w || !L.scales_f32 || !L.y || !shape_ok(L.rows, G.cols) || !aligned(L.w, 16) ||
                !aligned(L.scales_f32, 4) || !aligned(L.y, 4) || L.rows > INT32_MAX)
                return false;
        }
        next = G.first + G.n;
    }
    return next == n_lins;
}

ChLayout ch_layout(const fp8blk_linear* lins, int n_lins, const fp8blk_chain_group* groups, int n_groups,
                   std::vector<int64_t>* ll_of) {
    ChLayout l;
    std::vector<int64_t> off(n_lins, -1);
    int64_t words = 0, units = 0;
    for (int g = 0; g < n_groups; ++g) {
        if (groups[g].src >= 0 && off[groups[g].src] < 0) {
            off[groups[g].src] = words;
            words += (lins[groups[g].src].rows + 7) & ~INT64_C(7);  // 64-byte aligned runs
        }
        const int rpu = kChSlots / seg_slots((int)groups[g].cols);
        for (int j = groups[g].first; j < groups[g].first + groups[g].n; ++j) units += ceil_div(lins[j].rows, rpu);
    }
    l.units = units;
    l.ll_words = words;
    l.groups = kCtlBytes;
    l.recs = align64(l.groups + (size_t)n_groups * sizeof(ChGroup));
    l.ll = align64(l.recs + (size_t)units * sizeof(ChRec));
    l.total = align64(l.ll + (size_t)words * 8);
    if (ll_of) *ll_of = off;
    return l;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" size_t fp8blk_chain_bytes(const fp8blk_linear* linears, int n_linears, const fp8blk_chain_group* groups,
                                     int n_groups) {
    if (!ch_valid(linears, n_linears, groups, n_groups)) return 0;
    return ch_layout(linears, n_linears, groups, n_groups, nullptr).total;
}

extern "C" int fp8blk_chain_init(fp8blk_chain* ch, const fp8blk_linear* linears, int n_linears,
                                 const fp8blk_chain_group* groups, int n_groups, void* ws, size_t ws_bytes,
                                 fp8blk_stream_t stream) {
    if (!ch || !ch_valid(linears, n_linears, groups, n_groups)) return FP8BLK_ERR_ARG;
    std::vector<int64_t> ll_of;
    const ChLayout lay = ch_layout(linears, n_linears, groups, n_groups, &ll_of);
    if (lay.ll_words > INT32_MAX) return FP8BLK_ERR_ARG;
    if (!ws || !aligned(ws, 256) || ws_bytes < lay.total) return FP8BLK_ERR_WORKSPACE;
    std::vector<unsigned char> host(lay.ll, 0);
    ChGroup* gd = reinterpret_cast<ChGroup*>(host.data() + lay.groups);
    ChRec* rd = reinterpret_cast<ChRec*>(host.data() + lay.recs);
    int64_t u = 0;
    for (int g = 0; g < n_groups; ++g) {
        const fp8blk_chain_group& G = groups[g];
        gd[g].cols = (int32_t)G.cols;
        gd[g].src_ll = G.src >= 0 ? (int32_t)ll_of[G.src] : -1;
        gd[g].c = G.src >= 0 ? G.c : 1.0f;
        gd[g].pad = 0;
        const int rpu = kChSlots / seg_slots((int)G.cols);
        const int64_t GC = ceil_div(G.cols, kBlock);
        for (int j = G.first; j < G.first + G.n; ++j) {
            const fp8blk_linear& L = linears[j];
            for (int64_t r0 = 0; r0 < L.rows; r0 += rpu, ++u) {
                ChRec& r = rd[u];
                r.w = static_cast<const uint8_t*>(L.w) + r0 * G.cols;
                r.grid = L.scales_f32 + (r0 >> 7) * GC;
                r.y = L.y + r0;
                r.ll = ll_of[j] >= 0 ? (int32_t)(ll_of[j] + r0) : -1;
                r.left = (int32_t)std::min<int64_t>(rpu, L.rows - r0);
                r.cols = (int32_t)G.cols;
                r.group = g;
            }
        }
    }
    const int cus = device_cus();
    if (cus < 1) return FP8BLK_ERR_HIP;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    // descriptors, records and zeroed control words; the linked outputs start at epoch 0
    if (hipMemcpyAsync(ws, host.data(), host.size(), hipMemcpyHostToDevice, st) != hipSuccess) return FP8BLK_ERR_HIP;
    if (lay.ll_words > 0 &&
        hipMemsetAsync(static_cast<unsigned char*>(ws) + lay.ll, 0, (size_t)lay.ll_words * 8, st) != hipSuccess)
        return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FP8BLK_ERR_HIP;
    ch->plan = ws;
    ch->units = lay.units;
    ch->n_linears = n_linears;
    ch->n_groups = n_groups;
    ch->grid = cus;
    ch->reserved = 0;
    return FP8BLK_OK;
}

extern "C" int fp8blk_gemv_chain(const fp8blk_chain* ch, const uint16_t* x0_bf16, fp8blk_stream_t stream) {
    if (!ch || !ch->plan || ch->units < 1 || ch->grid < 1 || ch->n_linears < 1 || ch->n_groups < 1 || !x0_bf16 ||
        !aligned(x0_bf16, 16))
        return FP8BLK_ERR_ARG;
    unsigned char* ws = static_cast<unsigned char*>(ch->plan);
    const size_t recs = align64(kCtlBytes + (size_t)ch->n_groups * sizeof(ChGroup));
    ChArgs a;
    a.ctl = reinterpret_cast<uint32_t*>(ws);
    a.groups = reinterpret_cast<const ChGroup*>(ws + kCtlBytes);
    a.recs = reinterpret_cast<const ChRec*>(ws + recs);
    a.ll = reinterpret_cast<uint64_t*>(ws + align64(recs + (size_t)ch->units * sizeof(ChRec)));
    a.x0 = x0_bf16;
    a.units = ch->units;
    a.n_groups = ch->n_groups;
    (void)hipGetLastError();
    void* args[] = {&a};
    if (hipLaunchCooperativeKernel((const void*)k_chain, dim3((unsigned)ch->grid), dim3(kChWaves * kLanes), args, 0,
                                   reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return FP8BLK_ERR_HIP;
    return launch_status();
}

extern "C" int fp8blk_chain_status(const fp8blk_chain* ch, fp8blk_stream_t stream) {
    if (!ch || !ch->plan) return FP8BLK_ERR_ARG;
    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    uint32_t err = 0;
    uint32_t* ctl = static_cast<uint32_t*>(ch->plan);
    if (hipMemcpyAsync(&err, ctl + kCtlErr, 4, hipMemcpyDeviceToHost, st) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FP8BLK_ERR_HIP;
    if (err == 0) return FP8BLK_OK;
    const uint32_t zero = 0;
    if (hipMemcpyAsync(ctl + kCtlErr, &zero, 4, hipMemcpyHostToDevice, st) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(st) != hipSuccess) return FP8BLK_ERR_HIP;
    return FP8BLK_ERR_TIMEOUT;
}
