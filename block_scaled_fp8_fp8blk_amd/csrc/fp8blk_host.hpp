// Host-side argument checks shared by the entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

}  // namespace fp8blk
