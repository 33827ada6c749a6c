// mla_common.hpp -- LDS layout helpers and small device routines shared by the two MLA split
// kernels: mla_split.hip (score waves of 32 query rows) and mla_wide.hip (512-byte fp8 rows of
// one cache, score waves covering all 64 query rows).  The line and tail ring layout, its chunk permutations and the measured
// bank-conflict model they satisfy are described at the top of mla_split.hip.
#pragma once

#include "device_common.hpp"

namespace gqa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 64;            // query rows per CTA
constexpr int kThreads = 512;
constexpr int kLineSlots = 4;      // ring of the rows' first 512 bytes
constexpr int kTailSlots = 3;      // ring of the 64-byte rope tails (576-byte rows)
constexpr int kIdSlots = 4;        // ring of slot-id lists
constexpr int kNoMax = -(1 << 20); // integer maximum of a block with no visible key
// A row's reference maximum moves only when a block's maximum exceeds it by more than this, so
// that the running sums and accumulators are rarely rescaled; weights are then at most
// 2^(8 + kLazyMax).  Kept small: a block whose reference lags the other block's by more than 24
// loses its fp16 weights in the value waves' alignment, each at most 2^(kLazyMax + 1 - 24) of the
// row's largest.
constexpr int kLazyMax = 3;

// KV16: bf16 rows (1152 or 1024 bytes) in tiles of 32 keys, so that a tile's bytes (36 KiB for
// 576-wide rows) and the ring match those of 64 fp8 keys.
template <int DQK, bool KV16>
struct MlaLayout {
    static constexpr int kBK = KV16 ? 32 : 64;              // keys per tile
    static constexpr bool kTail = DQK == 576;               // rope tails in their own ring
    static constexpr int kTailOff = kLineSlots * 32768;
    static constexpr int kPOff = kTailOff + (kTail ? kTailSlots * 4096 : 0);
    static constexpr int kMlOff = kPOff + 2 * 8192;         // P [2][64 rows][64 keys] fp16
    static constexpr int kMlBytes = 2 * 256;                // m [blocks 0, 1][64 rows]
    static constexpr int kIdOff = kMlOff + 2 * kMlBytes;
    static constexpr int kBadOff = kIdOff + kIdSlots * 256;   // per tile: 64-bit mask of skipped keys
    static constexpr int kLdsBytes = kBadOff + kIdSlots * 8;
    static_assert(DQK == 576 || DQK == 512, "row width");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int swz_line(int pos) { return ((pos >> 2) & 1) | (pos & 2) | ((pos >> 1) & 4); }
__device__ __forceinline__ int swz_tail(int pos) { return (pos >> 2) & 3; }
// Byte offsets inside a line slot of 16-byte chunk c (< 8) of line `line`, and inside a tail slot
// of chunk c (< 4) of a rope tail.
__device__ __forceinline__ int line_off(int line, int pos, int c) {
    return line * 8192 + pos * 128 + ((c ^ swz_line(pos)) << 4);
}
__device__ __forceinline__ int tail_off(int pos, int c) { return pos * 64 + ((c ^ swz_tail(pos)) << 4); }
// Slot-list index (0..63, relative to the tile) of the key at tile position pos.
__device__ __forceinline__ int key_of_pos(int pos) { return 8 * (pos & 7) + (pos >> 3); }

// bf16 rows: a line slot holds the 128-byte lines j = 0..7 (elements 64 j .. 64 j + 63) of a
// tile's 32 keys, line j at j * 4096, tile position P at P * 128; a tail slot holds the 128-byte
// rope tails (elements 512 .. 575) the same way.  Chunks are permuted by an XOR with swz16(P)
// (bits 2, 3 and 1 of P): the score reads (16 lanes with one chunk index, keys of both parities
// of bits 1-3) and the transposed value reads (keys P .. P + 3, four chunks of one 64-byte half
// each; P and P + 2 land in opposite halves) touch distinct slots of a bank row.  Positions
// 8 i .. 8 i + 7 hold keys i, 4 + i, .., 28 + i of the tile.
__device__ __forceinline__ int swz16(int pos) { return ((pos >> 2) & 1) | ((pos >> 2) & 2) | ((pos << 1) & 4); }
__device__ __forceinline__ int line_off16(int line, int pos, int c) {
    return line * 4096 + pos * 128 + ((c ^ swz16(pos)) << 4);
}
__device__ __forceinline__ int key_of_pos16(int pos) { return 4 * (pos & 7) + (pos >> 3); }

// P rows of a tile: 128 bytes per query row (64 fp16 weights in tile-position order), the
// 16-byte slot q (weights 8 q .. 8 q + 7) stored at slot q ^ ((row >> 1) & 7).  The value waves'
// reads of one slot by 16 rows whose bits 1-3 differ (with either bit 0) then touch 16 distinct
// 16-byte slots of a 256-byte bank row.
__device__ __forceinline__ int p_slot(int row, int q) { return row * 128 + ((q ^ ((row >> 1) & 7)) << 4); }

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
// Two fp32 to packed fp16, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ f16x2 pack_f16x2(float a, float b) {
    f16x2 r;
    r.x = static_cast<_Float16>(a);
    r.y = static_cast<_Float16>(b);
    return r;
}
// Eight bf16 values (two transposed reads of four) to fp16: exact for magnitudes in fp16's
// normal range (every 8-bit significand fits in fp16's 11), rounded to nearest even below it (an
// error under 2^-25), infinite above 65504.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(s16x4 a, s16x4 b) {
    const u32x2 wa = __builtin_bit_cast(u32x2, a), wb = __builtin_bit_cast(u32x2, b);
    const f16x2 p0 = pack_f16x2(__uint_as_float(wa.x << 16), __uint_as_float(wa.x & 0xffff0000u));
    const f16x2 p1 = pack_f16x2(__uint_as_float(wa.y << 16), __uint_as_float(wa.y & 0xffff0000u));
    const f16x2 p2 = pack_f16x2(__uint_as_float(wb.x << 16), __uint_as_float(wb.x & 0xffff0000u));
    const f16x2 p3 = pack_f16x2(__uint_as_float(wb.y << 16), __uint_as_float(wb.y & 0xffff0000u));
    return f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
// Eight OCP e4m3fn bytes to fp16, exactly (every e4m3fn value is an fp16 value).
__device__ __forceinline__ f16x8 fp8x8_to_f16x8(uint32_t lo, uint32_t hi) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// Direct HBM -> LDS copies: lane L's bytes land at m0 + 16 L (or 4 L).  Every pool row is read
// once, so the copies are non-temporal (nt): on gfx950 that streaming hint lifts the bandwidth of
// gathers of random 576-byte rows by about a quarter over default-policy loads.
__device__ __forceinline__ void copy16(const uint8_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void copy4(const int32_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dword %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}
// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 31] (larger n waits for vmcnt(31)).
__device__ __forceinline__ void wait_vmem(int n) {
    switch (n) {
#define GQA_WAIT_CASE(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        GQA_WAIT_CASE(0) GQA_WAIT_CASE(1) GQA_WAIT_CASE(2) GQA_WAIT_CASE(3) GQA_WAIT_CASE(4)
        GQA_WAIT_CASE(5) GQA_WAIT_CASE(6) GQA_WAIT_CASE(7) GQA_WAIT_CASE(8) GQA_WAIT_CASE(9)
        GQA_WAIT_CASE(10) GQA_WAIT_CASE(11) GQA_WAIT_CASE(12) GQA_WAIT_CASE(13) GQA_WAIT_CASE(14)
        GQA_WAIT_CASE(15) GQA_WAIT_CASE(16) GQA_WAIT_CASE(17) GQA_WAIT_CASE(18) GQA_WAIT_CASE(19)
        GQA_WAIT_CASE(20) GQA_WAIT_CASE(21) GQA_WAIT_CASE(22) GQA_WAIT_CASE(23) GQA_WAIT_CASE(24)
        GQA_WAIT_CASE(25) GQA_WAIT_CASE(26) GQA_WAIT_CASE(27) GQA_WAIT_CASE(28) GQA_WAIT_CASE(29)
        GQA_WAIT_CASE(30)
#undef GQA_WAIT_CASE
        default: asm volatile("s_waitcnt vmcnt(31)" ::: "memory"); break;
    }
}

// Loads 8 bf16 query values at d (< DQK) of one row: the latent part from q, the rope part from
// q_pe.  8-element pieces never straddle the boundary (it is a multiple of 8).
template <int DLAT>
__device__ __forceinline__ u32x4 load_q8(const uint16_t *ql, const uint16_t *qp, int d) {
    return d < DLAT ? *reinterpret_cast<const u32x4 *>(ql + d)
                    : *reinterpret_cast<const u32x4 *>(qp + (d - DLAT));
}

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per 16-lane row of a 16x16 MFMA
// result), identical in all four: v_permlane32_swap and v_permlane16_swap hand back the values of
// both lanes of a pair.
__device__ __forceinline__ float rows4_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

}  // namespace
}  // namespace gqa
