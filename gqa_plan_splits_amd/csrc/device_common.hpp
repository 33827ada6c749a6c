// device_common.hpp -- small gfx950 device helpers shared by the split and reduce kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// Native vector types for data moves: HIP's uint4/uint2 structs are copied with memcpy, which
// can leave arrays of them on the stack instead of in registers.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;

// Eight OCP e4m3fn bytes (little-endian in lo, hi) to eight bf16 values, exactly: every e4m3
// value, subnormals included, is representable in bf16.  One v_cvt_scalef32_pk_bf16_fp8 per
// pair, with unit scale.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 bits to fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 to packed bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r.x = static_cast<__bf16>(a);
    r.y = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, r);
}

// Exchange with the lane whose index differs in bit 4 (mask 16) or bit 5 (mask 32).
__device__ __forceinline__ float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 4x4 byte transpose: y_e holds byte e of x0, x1, x2, x3 (in that order, low byte first).
// v_perm_b32 picks each result byte from the 8-byte pair {first operand: bytes 4-7, second
// operand: bytes 0-3}.
__device__ __forceinline__ void transpose4x4_bytes(uint32_t x0, uint32_t x1, uint32_t x2,
                                                   uint32_t x3, uint32_t &y0, uint32_t &y1,
                                                   uint32_t &y2, uint32_t &y3) {
    const uint32_t u0 = __builtin_amdgcn_perm(x1, x0, 0x05010400u);  // x0.0 x1.0 x0.1 x1.1
    const uint32_t u1 = __builtin_amdgcn_perm(x1, x0, 0x07030602u);  // x0.2 x1.2 x0.3 x1.3
    const uint32_t v0 = __builtin_amdgcn_perm(x3, x2, 0x05010400u);  // x2.0 x3.0 x2.1 x3.1
    const uint32_t v1 = __builtin_amdgcn_perm(x3, x2, 0x07030602u);  // x2.2 x3.2 x2.3 x3.3
    y0 = __builtin_amdgcn_perm(v0, u0, 0x05040100u);                 // x0.0 x1.0 x2.0 x3.0
    y1 = __builtin_amdgcn_perm(v0, u0, 0x07060302u);                 // x0.1 x1.1 x2.1 x3.1
    y2 = __builtin_amdgcn_perm(v1, u1, 0x05040100u);                 // x0.2 x1.2 x2.2 x3.2
    y3 = __builtin_amdgcn_perm(v1, u1, 0x07060302u);                 // x0.3 x1.3 x2.3 x3.3
}

// Workgroups are dispatched round-robin over the 8 XCDs (hardware id % 8).  Remap so that each
// XCD receives a contiguous range of logical work items: neighbouring items (which read the
// same keys) then share that XCD's L2.  Returns -1 for the padding ids of the last range.
__device__ __forceinline__ int xcd_logical_block(int hw_id, int total) {
    const int per_xcd = (total + 7) >> 3;
    const int logical = (hw_id & 7) * per_xcd + (hw_id >> 3);
    return logical < total ? logical : -1;
}

inline int xcd_grid_size(int total) { return ((total + 7) >> 3) << 3; }

// Length-proportional partitions: request b owns partition slots part_start[b] ..
// part_start[b + 1] - 1 (part_start non-decreasing, part_start[0] = 0).  Returns the request
// owning slot i, or batch when i lies past the last slot.  Every lane of the wave takes part
// (one load per 64 requests) and gets the same, wave-uniform, answer.
__device__ __forceinline__ int request_of_slot(const int32_t *part_start, int batch, int i) {
    const int lane = threadIdx.x & 63;
    int b = 0;
    for (int j0 = 1; j0 <= batch; j0 += 64) {
        const int j = j0 + lane;
        const bool le = j <= batch && part_start[j] <= i;
        b += __builtin_popcountll(__builtin_amdgcn_ballot_w64(le));
    }
    return __builtin_amdgcn_readfirstlane(b);
}

}  // namespace gqa
