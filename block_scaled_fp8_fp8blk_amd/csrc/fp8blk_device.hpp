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

// e8m0 code -> f32 by building the exponent field: code c >= 1 is the normal
// f32 2^(c-127) with exponent field c; code 0 is 2^-127, the f32 subnormal
// with only mantissa bit 22 set. (0xFF, refused at load, would give +inf.)
__device__ __forceinline__ float e8m0_to_f32(uint32_t c) {
    return as_f32(c ? (c << 23) : 0x00400000u);
}

// An e8m0 code as the scale operand of gfx950's scaled conversions
// (v_cvt_scalef32_*). Those read only the exponent field of their f32 scale
// and multiply by 2^(field - 127): measured over every code byte of the FP4
// and FP8 conversions, a scale of 0.0, -0.0 or any f32 subnormal acts as
// 2^-127, 1.5 and -1.0 act as 1.0. So byte k of a dword of codes, moved into
// the exponent field (bits 23..30) by one shift, is its scale, code 0 (2^-127)
// included, whatever the shift leaves in the sign and mantissa bits.
template <int K>
__device__ __forceinline__ float e8m0_cvt_scale(uint32_t d) {
    static_assert(K >= 0 && K < 4, "byte of a dword");
    return as_f32(K < 3 ? d << (23 - 8 * K) : d >> 1);
}

// Exchange lane bit 3 with the index of a register pair (x, y) inside each row
// of 16 lanes: x'[l] = bit 3 of l ? y[l ^ 8] : x[l], y'[l] = bit 3 of l ? y[l]
// : x[l ^ 8]. Each is one DPP move (rotate the row by 8) whose bank mask
// writes only the lanes that change (banks 2 and 3 are lanes 8..15 of a row);
// the other lanes keep the old value.
__device__ __forceinline__ void swap_lane_bit3(uint32_t& x, uint32_t& y) {
    const uint32_t nx = (uint32_t)__builtin_amdgcn_update_dpp((int)x, (int)y, 0x128, 0xF, 0xC, false);
    const uint32_t ny = (uint32_t)__builtin_amdgcn_update_dpp((int)y, (int)x, 0x128, 0xF, 0x3, false);
    x = nx;
    y = ny;
}

// Exchange the upper 32 lanes of a with the lower 32 lanes of b, dword by
// dword (permlane32_swap): afterwards a[l] = l < 32 ? a[l] : b[l - 32] and
// b[l] = l < 32 ? a[l + 32] : b[l]. The bf16 slab kernels load 16-byte pieces
// so that each load instruction reads whole lines; this swap then hands lane
// l the two halves of its own 32-byte chunk.
__device__ __forceinline__ void swap_lane_halves(uint4& a, uint4& b) {
    uint32_t* pa = reinterpret_cast<uint32_t*>(&a);
    uint32_t* pb = reinterpret_cast<uint32_t*>(&b);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const auto r = __builtin_amdgcn_permlane32_swap(pa[d], pb[d], false, false);
        pa[d] = r[0];
        pb[d] = r[1];
    }
}

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

// The same values through gfx950's scaled conversion v_cvt_scalef32_pk_f32_fp8,
// which multiplies by the (power-of-two) scale inside the conversion: one
// instruction per two codes instead of three. Measured exact, against the
// exact products, for all 254 finite codes x all 255 scale codes, including
// f32 subnormal results.
__device__ __forceinline__ void decode4_fp8_scaled(uint32_t d, float s, float* w) {
    const v2f lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, s, false);  // bytes 0, 1
    const v2f hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(d, s, true);   // bytes 2, 3
    w[0] = lo.x;
    w[1] = lo.y;
    w[2] = hi.x;
    w[3] = hi.y;
}

__device__ __forceinline__ void decode16_fp8_scaled(const uint4& c, float s, float* w) {
    decode4_fp8_scaled(c.x, s, w + 0);
    decode4_fp8_scaled(c.y, s, w + 4);
    decode4_fp8_scaled(c.z, s, w + 8);
    decode4_fp8_scaled(c.w, s, w + 12);
}

// 16-byte load that streams past the caches' retention (the weights are read
// once per call): global_load_dwordx4 with the nontemporal hint.
// The pointer is taken as a global-memory address (every buffer of this
// library is device global memory), so the load is a global_load and not a
// flat one, which would also hold the scalar-load counter.
typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const v4u global_v4u;
typedef __attribute__((address_space(1))) const float global_f32;
typedef __attribute__((address_space(1))) float global_f32_out;
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    const v4u v = __builtin_nontemporal_load((global_v4u*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
// Plain (cached) global loads and stores of the same kind.
__device__ __forceinline__ uint4 load_global16(const void* p) {
    const v4u v = *(global_v4u*)p;
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float load_global_f32(const float* p) { return *(global_f32*)p; }
__device__ __forceinline__ void store_global_f32(float* p, float v) { *(global_f32_out*)p = v; }

// Two bf16 patterns packed in a dword (lower column in the low half) widened
// to f32: a bf16 pattern is the high half of the f32.
__device__ __forceinline__ void widen2_bf16(uint32_t d, float* w) {
    w[0] = as_f32(d << 16);
    w[1] = as_f32(d & 0xffff0000u);
}

// bf16 of the f32 product c * v, rounded to nearest even (NaN: the quiet NaN):
// the input a dependent linear reads from an earlier linear's f32 output.
__device__ __forceinline__ uint32_t bf16_of_scaled(float c, uint32_t vbits) {
    const float f = c * as_f32(vbits);
    const uint32_t u = as_u32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void widen8_bf16(const uint4& v, float* w) {
    widen2_bf16(v.x, w + 0);
    widen2_bf16(v.y, w + 2);
    widen2_bf16(v.z, w + 4);
    widen2_bf16(v.w, w + 6);
}

// DPP lane permutations inside a row of 16 lanes. row_ror:8 reads lane l ^ 8;
// once values are equal across that pairing, row_ror:4 pairs l with l ^ 4 as
// values; quad_perm [2,3,0,1] reads l ^ 2 and [1,0,3,2] reads l ^ 1.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return as_f32((uint32_t)__builtin_amdgcn_update_dpp(0, (int)as_u32(v), CTRL, 0xF, 0xF, false));
}
constexpr int kRowRor8 = 0x128, kRowRor4 = 0x124, kQuadXor2 = 0x4E, kQuadXor1 = 0xB1;

// v + (v of the lane differing in bit 5): permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second.
__device__ __forceinline__ float bfly32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(as_u32(v), as_u32(v), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
}
// v + (v of the lane differing in bit 4): permlane16_swap exchanges the odd
// rows of its first operand with the even rows of its second.
__device__ __forceinline__ float bfly16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(as_u32(v), as_u32(v), false, false);
    return as_f32(r[0]) + as_f32(r[1]);
}
// The bit 3..0 levels of the tree inside each row of 16 lanes.
__device__ __forceinline__ float tree_row16(float v) {
    v = v + dpp<kRowRor8>(v);
    v = v + dpp<kRowRor4>(v);
    v = v + dpp<kQuadXor2>(v);
    v = v + dpp<kQuadXor1>(v);
    return v;
}

// Four independent 64-lane trees at once (a transposing reduction): the bit 5
// and bit 4 levels each exchange half of two registers and add, so after them
// one register holds value k's partial sums in row kRowOf4[k]; the last four
// levels run inside the rows. Each value gets exactly the tree of tree64.
// Returns the register holding, in every lane of row kRowOf4[k], sum k.
constexpr int kRowOf4[4] = {0, 2, 1, 3};
__device__ __forceinline__ float tree64x4(float v0, float v1, float v2, float v3) {
    const auto a = __builtin_amdgcn_permlane32_swap(as_u32(v0), as_u32(v1), false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(as_u32(v2), as_u32(v3), false, false);
    const float s01 = as_f32(a[0]) + as_f32(a[1]);  // lanes 0-31: v0, lanes 32-63: v1
    const float s23 = as_f32(b[0]) + as_f32(b[1]);  // lanes 0-31: v2, lanes 32-63: v3
    const auto c = __builtin_amdgcn_permlane16_swap(as_u32(s01), as_u32(s23), false, false);
    const float u = as_f32(c[0]) + as_f32(c[1]);    // rows 0..3: v0, v2, v1, v3
    return tree_row16(u);
}
// V independent 64-lane trees (V a multiple of 4), four per output register:
// out[k] holds, in every lane of row kRowOf4[j], the sum of value 4k + j.
template <int V>
__device__ __forceinline__ void tree64xV(const float* v, float* out) {
    static_assert(V % 4 == 0, "groups of four");
#pragma unroll
    for (int k = 0; k < V / 4; ++k) out[k] = tree64x4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
}

__device__ __forceinline__ float lane_value(float v, int lane) {
    return as_f32((uint32_t)__builtin_amdgcn_readlane((int)as_u32(v), lane));
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

// Workgroups are dealt to the 8 XCDs of the chip in turn (workgroup b runs
// on XCD b % 8). This renumbering gives each XCD a contiguous range of
// numbers, so that a persistent kernel whose waves take consecutive work
// units by number keeps each XCD on contiguous runs of units (its L2 then
// serves the activations and scale rows of fewer linears at a time). A
// bijection on [0, gridDim.x) for every grid size.
__device__ __forceinline__ int xcd_contiguous_block() {
    const int G = gridDim.x, wg = blockIdx.x, xcd = wg % 8, q = G / 8, r = G % 8;
    return xcd * q + min(xcd, r) + wg / 8;
}

}  // namespace fp8blk
