// Device helpers shared by the FP8-blk kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kLanes = 64;                    // wavefront width
constexpr int kChunk = 16;                    // columns per lane per segment (one 16-byte code load)
constexpr int kSegCols = kLanes * kChunk;     // 1024 columns per segment
constexpr int kBlock = 128;                   // scale block edge

__device__ __forceinline__ float as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Four e4m3 codes (little-endian bytes of d, lowest column first) times a
// power-of-two block scale. gfx950's v_cvt_pk_f32_fp8 reads OCP E4M3 and is
// exact (every e4m3 value is an f32 value); the product by a power of two is
// exact for every weight the load check accepts (bf16 values are f32 values).
__device__ __forceinline__ void decode4_fp8(uint32_t d, float s, float* w) {
    const v2f lo = __builtin_amdgcn_cvt_pk_f32_fp8(d, false);  // bytes 0, 1
    const v2f hi = __builtin_amdgcn_cvt_pk_f32_fp8(d, true);   // bytes 2, 3
    w[0] = lo.x * s;
    w[1] = lo.y * s;
    w[2] = hi.x * s;
    w[3] = hi.y * s;
}

__device__ __forceinline__ void decode16_fp8(const uint4& c, float s, float* w) {
    decode4_fp8(c.x, s, w + 0);
    decode4_fp8(c.y, s, w + 4);
    decode4_fp8(c.z, s, w + 8);
    decode4_fp8(c.w, s, w + 12);
}

// Two bf16 patterns packed in a dword (lower column in the low half) widened
// to f32: a bf16 pattern is the high half of the f32.
__device__ __forceinline__ void widen2_bf16(uint32_t d, float* w) {
    w[0] = as_f32(d << 16);
    w[1] = as_f32(d & 0xffff0000u);
}

__device__ __forceinline__ void widen8_bf16(const uint4& v, float* w) {
    widen2_bf16(v.x, w + 0);
    widen2_bf16(v.y, w + 2);
    widen2_bf16(v.z, w + 4);
    widen2_bf16(v.w, w + 6);
}

// Sum of one value per lane over the 64 lanes, as a pairwise tree that pairs
// lanes differing in bit 5 first, then bit 4, ..., bit 0. Every lane ends
// with the same bits (IEEE addition is commutative).
__device__ __forceinline__ float tree64(float v) {
    v = v + __shfl_xor(v, 32);
    v = v + __shfl_xor(v, 16);
    v = v + __shfl_xor(v, 8);
    v = v + __shfl_xor(v, 4);
    v = v + __shfl_xor(v, 2);
    v = v + __shfl_xor(v, 1);
    return v;
}

}  // namespace fp8blk
