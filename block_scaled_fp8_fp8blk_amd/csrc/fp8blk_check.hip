// Load-time check, scale-grid decode and the bf16 dequant slab.
//
// "Module dsv4_gpu" page (memra-engine docs), struct Fp8Dense: e8m0 block
// scales are powers of two decoded to f32 once at load, and a 0xFF scale is
// refused there. Same page, rungs paragraph: dequantization to bf16 refuses
// any element that is not exactly a bf16 value. Same page, DenseBf16: the
// dequant slab holds exactly those bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fp8blk.h"
#include "fp8blk_device.hpp"
#include "fp8blk_host.hpp"

namespace fp8blk {
namespace {

constexpr uint64_t kNone = ~0ull;
constexpr int kThreads = 256;

__global__ void k_verdict_init(unsigned long long* v) {
    if (threadIdx.x < 3) v[threadIdx.x] = kNone;
}

__global__ void k_scales(const uint8_t* __restrict__ s, int64_t n, float* __restrict__ out,
                         unsigned long long* __restrict__ verdict) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const uint32_t c = s[i];
        out[i] = e8m0_to_f32(c);
        if (c == 0xFFu) atomicMin(&verdict[0], (unsigned long long)i);
    }
}

// Is e4m3(b) * 2^(s - 127) exactly a finite bf16 value? Integer reasoning on
// the significand: the value is sig * 2^e with sig <= 15 (at most 4 bits),
// so it is representable iff its leading bit is at most 2^127 (bf16's top
// binade; 15 * 2^124 is below the largest finite bf16) and its lowest set
// bit is at least 2^-133 (bf16's subnormal spacing).
__device__ __forceinline__ bool exact_in_bf16(uint32_t b, uint32_t s) {
    const uint32_t E = (b >> 3) & 15u, m = b & 7u;
    const uint32_t sig = E ? (8u | m) : m;
    if (sig == 0) return true;
    const int e = (E ? (int)E - 10 : -9) + (int)s - 127;
    const int top = e + (31 - __clz(sig));
    const int low = e + (__ffs(sig) - 1);
    return top <= 127 && low >= -133;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
    for (int h = 32; h >= 1; h >>= 1) {
        const unsigned long long o = __shfl_xor(v, h);
        v = o < v ? o : v;
    }
    return v;
}

// One 16-code chunk per thread per step: NaN codes and inexact elements, each
// reported by its lowest row-major element index.
__global__ void k_codes(const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
                        int64_t rows, int64_t K, int64_t GC, unsigned long long* __restrict__ verdict) {
    const int64_t cpr = K / kChunk;  // chunks per row
    const int64_t n = rows * cpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    // The loop bound depends on the block only, so every lane of a wave runs
    // the same number of iterations (the wave-wide shuffles need all 64).
    for (int64_t b = blockIdx.x * (int64_t)blockDim.x; b < n; b += stride) {
        const int64_t g = b + threadIdx.x;
        unsigned long long nan_at = kNone, inexact_at = kNone;
        if (g < n) {
            const int64_t r = g / cpr, c0 = (g - r * cpr) * kChunk;
            const uint4 v = *reinterpret_cast<const uint4*>(codes + r * K + c0);
            const uint32_t s = scales[(r >> 7) * GC + (c0 >> 7)];
            const uint32_t d[4] = {v.x, v.y, v.z, v.w};
            for (int k = 15; k >= 0; --k) {
                const uint32_t byte = (d[k >> 2] >> (8 * (k & 3))) & 0xffu;
                const unsigned long long at = (unsigned long long)(r * K + c0 + k);
                if ((byte & 0x7fu) == 0x7fu)
                    nan_at = at;
                else if (!exact_in_bf16(byte, s))
                    inexact_at = at;
            }
        }
        if (__ballot(nan_at != kNone)) {
            const unsigned long long w = wave_min_u64(nan_at);
            if ((threadIdx.x & 63) == 0) atomicMin(&verdict[1], w);
        }
        if (__ballot(inexact_at != kNone)) {
            const unsigned long long w = wave_min_u64(inexact_at);
            if ((threadIdx.x & 63) == 0) atomicMin(&verdict[2], w);
        }
    }
}

// bf16 dequant slab: one 16-code chunk per thread per step. The f32 product
// gfx950's v_cvt_scalef32_pk_bf16_fp8 forms e4m3(code) * scale and rounds it
// to bf16: for an accepted element the product is a bf16 value, so the result
// is exact (the exhaustive code x scale table is checked against the oracle).
// Each thread takes U chunks of 16 codes per pass, chunks blockDim apart, all
// loads first; IDX is the index type (32-bit while rows * cols / 16 fits).
template <typename IDX, int U>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* __restrict__ codes,
                                                      const float* __restrict__ grid, IDX rows, IDX cpr, IDX GC,
                                                      uint16_t* __restrict__ out) {
    const IDX n = rows * cpr;
    const IDX step = (IDX)gridDim.x * blockDim.x * U;
    for (IDX g0 = (IDX)blockIdx.x * blockDim.x * U + threadIdx.x; g0 < n; g0 += step) {
        uint4 v[U];
        float sc[U];
        IDX r[U], c[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const IDX g = min(g0 + (IDX)u * blockDim.x, n - 1);  // a chunk past the end repeats the last one
            r[u] = g / cpr;
            c[u] = (g - r[u] * cpr) * kChunk;
            v[u] = load_stream16(codes + (int64_t)g * kChunk);
            sc[u] = load_global_f32(grid + (r[u] >> 7) * GC + (c[u] >> 7));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (g0 + (IDX)u * blockDim.x >= n) break;
            const uint32_t d[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
            uint32_t o[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                o[2 * k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], sc[u], false));
                o[2 * k + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(d[k], sc[u], true));
            }
            uint4* dst = reinterpret_cast<uint4*>(out + ((int64_t)r[u] * cpr * kChunk + c[u]));
            dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
            dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
        }
    }
}

int grid_for(int64_t work, int64_t cap) {
    int64_t b = ceil_div(work, kThreads);
    if (b > cap) b = cap;
    return (int)(b < 1 ? 1 : b);
}

// The load check's three verdict slots, run on a caller's buffer of at least
// fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK) bytes. k_verdict_init clears
// them first (a kernel, not a memset), so the buffer's earlier contents never
// matter.
int run_load_check(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows, int64_t cols,
                   float* scales_f32_out, unsigned long long* verdict, int64_t* first_bad, hipStream_t s) {
    (void)hipGetLastError();
    const int64_t GR = ceil_div(rows, kBlock), GC = ceil_div(cols, kBlock);
    k_verdict_init<<<1, 64, 0, s>>>(verdict);
    k_scales<<<grid_for(GR * GC, 1024), kThreads, 0, s>>>(scales_e8m0, GR * GC, scales_f32_out, verdict);
    k_codes<<<grid_for(rows * (cols / kChunk), 8192), kThreads, 0, s>>>(codes, scales_e8m0, rows, cols, GC,
                                                                       verdict);
    if (launch_status() != FP8BLK_OK) return FP8BLK_ERR_HIP;
    unsigned long long host[3] = {kNone, kNone, kNone};
    if (hipMemcpyAsync(host, verdict, sizeof host, hipMemcpyDeviceToHost, s) != hipSuccess) return FP8BLK_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return FP8BLK_ERR_HIP;
    const int kinds[3] = {FP8BLK_ERR_SCALE_FF, FP8BLK_ERR_NAN_CODE, FP8BLK_ERR_INEXACT};
    for (int k = 0; k < 3; ++k)
        if (host[k] != kNone) {
            if (first_bad) *first_bad = (int64_t)host[k];
            return kinds[k];
        }
    return FP8BLK_OK;
}

// Scratch of fp8blk_load_check_noalloc: the verdict slots in a static device
// array, one copy per GPU, held until the process ends. Host code never passes
// `scratch` itself to a kernel (on the host the name is only a stand-in): it
// passes the device address that hipGetSymbolAddress returns for the current
// device, looked up once per device and kept here.
constexpr size_t kScratchBytes = 256;
constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned long long scratch[kScratchBytes / sizeof(unsigned long long)];

std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, or NULL (HIP error).
void* scratch_for_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        p = q;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace
}  // namespace fp8blk

using namespace fp8blk;

extern "C" int fp8blk_abi_version(void) { return 1; }

extern "C" const char* fp8blk_strerror(int status) {
    switch (status) {
        case FP8BLK_OK: return "ok";
        case FP8BLK_ERR_ARG: return "invalid argument (null pointer, shape, alignment or M)";
        case FP8BLK_ERR_SCALE_FF: return "scale code 0xFF refused";
        case FP8BLK_ERR_NAN_CODE: return "NaN e4m3 code (0x7F or 0xFF) refused";
        case FP8BLK_ERR_INEXACT: return "element is not exactly a bf16 value";
        case FP8BLK_ERR_WORKSPACE: return "workspace missing or too small";
        case FP8BLK_ERR_HIP: return "HIP runtime error";
        case FP8BLK_ERR_BAD_SCALE: return "negative or NaN NVFP4 block scale refused";
        case FP8BLK_ERR_TIMEOUT: return "chained launch stopped waiting for an earlier group's outputs";
        default: return "unknown status";
    }
}

extern "C" size_t fp8blk_workspace_bytes(int op, int64_t rows, int64_t cols, int64_t M) {
    (void)M;
    switch (op) {
        case FP8BLK_OP_LOAD_CHECK: return 256;  // three 64-bit verdict slots, padded
        case FP8BLK_OP_DEQUANT_BF16: return 0;
        case FP8BLK_OP_GEMV: return 0;
        case FP8BLK_OP_BF16_TWIN: return 0;
        case FP8BLK_OP_GEMM_STAGED:
        case FP8BLK_OP_BF16_GEMM: return gemm_workspace_bytes(op, rows, cols);
        default: return 0;
    }
}

extern "C" int fp8blk_load_check(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows,
                                 int64_t cols, float* scales_f32_out, void* ws, size_t ws_bytes,
                                 int64_t* first_bad, fp8blk_stream_t stream) {
    if (first_bad) *first_bad = -1;
    if (!codes || !scales_e8m0 || !scales_f32_out || !shape_ok(rows, cols) || !aligned(codes, 16) ||
        !aligned(scales_f32_out, 4))
        return FP8BLK_ERR_ARG;
    if (!ws || ws_bytes < fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK, rows, cols, 1) || !aligned(ws, 8))
        return FP8BLK_ERR_WORKSPACE;
    return run_load_check(codes, scales_e8m0, rows, cols, scales_f32_out, static_cast<unsigned long long*>(ws),
                          first_bad, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_load_check_noalloc(const uint8_t* codes, const uint8_t* scales_e8m0, int64_t rows,
                                         int64_t cols, float* scales_f32_out, int64_t* first_bad,
                                         fp8blk_stream_t stream) {
    if (first_bad) *first_bad = -1;
    if (!codes || !scales_e8m0 || !scales_f32_out || !shape_ok(rows, cols) || !aligned(codes, 16) ||
        !aligned(scales_f32_out, 4))
        return FP8BLK_ERR_ARG;
    if (fp8blk_workspace_bytes(FP8BLK_OP_LOAD_CHECK, rows, cols, 1) > kScratchBytes) return FP8BLK_ERR_WORKSPACE;
    void* verdict = scratch_for_current_device();
    if (!verdict) return FP8BLK_ERR_HIP;
    return run_load_check(codes, scales_e8m0, rows, cols, scales_f32_out, static_cast<unsigned long long*>(verdict),
                          first_bad, reinterpret_cast<hipStream_t>(stream));
}

extern "C" int fp8blk_dequant_bf16(const uint8_t* codes, const float* scales_f32, int64_t rows, int64_t cols,
                                   uint16_t* out_bf16, fp8blk_stream_t stream) {
    if (!codes || !scales_f32 || !out_bf16 || !shape_ok(rows, cols) || !aligned(codes, 16) ||
        !aligned(out_bf16, 16) || !aligned(scales_f32, 4))
        return FP8BLK_ERR_ARG;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const int64_t GC = ceil_div(cols, kBlock), cpr = cols / kChunk, n = rows * cpr;
    constexpr int U = 4;
    const int blocks = grid_for(ceil_div(n, U), 8192);
    if (n < (INT64_C(1) << 31))
        k_dequant<uint32_t, U><<<blocks, kThreads, 0, s>>>(codes, scales_f32, (uint32_t)rows, (uint32_t)cpr,
                                                           (uint32_t)GC, out_bf16);
    else
        k_dequant<uint64_t, U><<<blocks, kThreads, 0, s>>>(codes, scales_f32, (uint64_t)rows, (uint64_t)cpr,
                                                           (uint64_t)GC, out_bf16);
    return launch_status();
}
