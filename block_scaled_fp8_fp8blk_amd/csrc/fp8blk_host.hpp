// Host-side argument checks shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "fp8blk.h"

namespace fp8blk {

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// rows >= 1, cols in [16, FP8BLK_MAX_COLS] and a multiple of 16, rows * cols
// representable.
inline bool shape_ok(int64_t rows, int64_t cols) {
    if (rows < 1 || cols < FP8BLK_MIN_COLS || cols > FP8BLK_MAX_COLS || (cols % 16) != 0)
        return false;
    return rows <= (INT64_C(1) << 46) / cols;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Launch-error status after enqueueing kernels.
inline int launch_status() {
    return hipGetLastError() == hipSuccess ? FP8BLK_OK : FP8BLK_ERR_HIP;
}

// Sequence launches (fp8blk_seq.hip, fp8blk_mfma.hip). A plan in the
// caller's workspace: n descriptors of kSeqDescBytes, then two arrays of
// n + 1 int64 prefix sums of work units.
constexpr int kSeqWaves = 4;         // waves per workgroup of the persistent kernels
constexpr int kSeqDescBytes = 64;    // one descriptor: one scalar load
constexpr int kMfSeqBlocksPerCU = 2; // workgroups per compute unit, matrix-core sequence
// The FP8 arm's kernels for panels of fewer than 8 rows hold no outputs in LDS
// and use at most 170 registers (three waves per SIMD): three workgroups per
// compute unit, 1.5 times the loads in flight. Measured on the whole-step
// sweep: M = 2 from 78.4 to 81.0 % of HBM peak, M = 4 from 74.8 to 77.3 %.
constexpr int kMfSeqSmallBlocksPerCU = 3;
constexpr int mf_seq_blocks_per_cu(bool fp8, int64_t M) { return fp8 && M < 8 ? kMfSeqSmallBlocksPerCU : kMfSeqBlocksPerCU; }
inline size_t plan_bytes(int n) { return (size_t)n * kSeqDescBytes + (size_t)(n + 1) * 2 * sizeof(int64_t); }

// LDS bytes a workgroup reserves (and leaves unused) so that no compute unit
// (160 KB of LDS) holds more than `per_cu` of them: a persistent kernel that
// deals its units to the waves in a fixed rotation assumes every wave
// progresses at the same rate.
constexpr int lds_cap_bytes(int per_cu) { return 160 * 1024 / (per_cu + 1) + 1024; }

// Compute units of the current device (-1 on a HIP error), looked up once per
// device.
inline int device_cus() {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < kMaxDev && (cus = cache[dev].load(std::memory_order_relaxed)) > 0) return cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < kMaxDev) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

// Writes the matrix-core sequence plan of n validated linears (panel rows M,
// the same for all) into host (plan_bytes(n) bytes); returns its work units.
int64_t mf_sequence_plan(unsigned char* host, bool fp8, const fp8blk_seq_linear* linears, int n);

// Workspace of the staged prefill GEMM (fp8blk_gemm.hip): the bf16 slab (for
// FP8BLK_OP_GEMM_STAGED) plus the library GEMM's workspace; 0 for a bad shape.
size_t gemm_workspace_bytes(int op, int64_t rows, int64_t cols);

}  // namespace fp8blk
