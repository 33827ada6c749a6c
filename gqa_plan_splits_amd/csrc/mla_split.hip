// mla_split.hip -- split kernel of absorbed MLA decode for gfx950.
//
// What it computes (moonmath-amd README, "MLA decode"; Modular MAX planner page, MLA-style
// bullet): every key row of the pool is one fused fp8 e4m3 row that serves as K (all DQK bytes)
// and as V (its first DV bytes), dequantized with one per-tensor kv_scale.  A CTA owns up to 64
// query rows of one request and walks one partition of that request's keys, writing the
// partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Work split (512 threads = 8 waves, one CTA per CU; waves w and w + 4 share SIMD w):
//   - Score waves 0-3: wave w computes S^T = K Q^T for query rows 32 (w & 1) .. +31 against tile
//     keys 32 (w >> 1) .. +31 on the block-scaled fp8 MFMA v_mfma_scale_f32_32x32x64_f8f6f4 (unit
//     scales), then the block's softmax.  K is used as stored.  A bf16 query row, scaled by a power
//     of two so its largest element lies in [128, 256), is the exact sum of two e4m3 vectors (hi =
//     nearest, lo = remainder) except below e4m3's subnormal step; each product runs twice.  The
//     block maximum is kept as an integer (the ceiling of the base-2 score), so probabilities of
//     different blocks differ by exact powers of two; they go to LDS as fp8 hi/lo pairs of
//     p * 2^8 (p <= 1), with the block maximum and two block sums: of the quantized probabilities
//     (the weights PV applies, which normalize the output, so that a dominant key carries no
//     quantization error into it) and of the exact ones (which give the log-sum-exp).
//   - Value waves 4-7: wave 4 + v accumulates output columns 128 v .. +127 (line v of the key rows)
//     for all 64 rows on the same MFMA: V^T comes from the fp8 tile through ds_read_b64_tr_b8, P^T
//     from LDS, and the power of two that aligns each 32-key block with the row's running maximum
//     is the MFMA's per-lane B scale.  The value waves also move the data: wave 4 + v copies line v
//     of every key of a tile (and a quarter of the 64-byte rope tails of 576-byte rows) straight
//     from HBM into LDS with global_load_lds_dwordx4, two tiles ahead, after loading the tile's
//     slot ids the same way two tiles before that.  The copies are issued from inline assembly and
//     waited for with explicit vmcnt counts (the compiler would drain every copy in flight before
//     each LDS read).
//   - One barrier per tile: in step t the score waves work on tile t while the value waves apply
//     tile t - 1, so on each SIMD the MFMAs of one role overlap the vector work of the other.
//
// LDS tile (one slot of a three-slot ring): line j (bytes 128 j .. 128 j + 127 of the key rows) of
// the 64 keys fills 8 KiB at j * 8192, tile position P at P * 128, its 16-byte chunks permuted by
// an XOR with (P >> 1) & 7; the 64-byte rope tails of 576-byte rows fill 4 KiB at 32768, position
// P at P * 64, chunks permuted with (P >> 2) & 3.  A copy instruction writes 1 KiB of consecutive
// 16-byte slots, so it moves whole 128-byte lines: one line of 8 keys (positions 8 i .. 8 i + 7
// hold keys i, 8 + i, .., 56 + i of the tile, so that each lane's keys over the 8 instructions are
// consecutive in the slot list), or 16 rope tails.  With these permutations the score-operand
// reads, the transposed value reads (whose two 16-column halves take chunks c and c ^ 4) and the
// copies are free of bank conflicts.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kBM = 64;            // query rows per CTA
constexpr int kBK = 64;            // keys per tile
constexpr int kThreads = 512;
constexpr int kSlots = 3;          // LDS tile ring
constexpr int kIdSlots = 4;        // per value wave: ring of slot-id lists
constexpr int kNoMax = -(1 << 20); // integer maximum of a block with no visible key

template <int DQK>
struct MlaLayout {
    static constexpr int kSteps = DQK / 64;               // 64-byte contraction steps per row
    static constexpr bool kTail = DQK == 576;             // rope tails in their own region
    static constexpr int kSlotBytes = 32768 + (kTail ? 4096 : 0);
    static constexpr int kPOff = kSlots * kSlotBytes;     // P [2 buffers][hi, lo][64 rows][64 keys]
    static constexpr int kMlOff = kPOff + 2 * 2 * 4096;   // ML [2][64 rows][2 blocks][m, lq, le, -]
    static constexpr int kIdOff = kMlOff + 2 * 2048;      // ids [4 value waves][4][64]
    static constexpr int kLdsBytes = kIdOff + 4 * kIdSlots * 256;
    static constexpr int kCopies = 8 + (kTail ? 1 : 0);   // copy instructions per tile per wave
    static_assert(DQK == 576 || DQK == 512, "row width");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int swz_line(int pos) { return (pos >> 1) & 7; }
__device__ __forceinline__ int swz_tail(int pos) { return (pos >> 2) & 3; }
// Byte offsets inside a tile slot of 16-byte chunk c of a line (c < 8) or of a rope tail (c < 4).
__device__ __forceinline__ int line_off(int line, int pos, int c) {
    return line * 8192 + pos * 128 + ((c ^ swz_line(pos)) << 4);
}
__device__ __forceinline__ int tail_off(int pos, int c) {
    return 32768 + pos * 64 + ((c ^ swz_tail(pos)) << 4);
}
// Slot-list index (0..63, relative to the tile) of the key at tile position pos.
__device__ __forceinline__ int key_of_pos(int pos) { return 8 * (pos & 7) + (pos >> 3); }

// Direct HBM -> LDS copies: lane L's bytes land at m0 + 16 L (or 4 L).  Every pool row is read
// once, so the copies are non-temporal (nt): on gfx950 that streaming hint lifts the bandwidth of
// gathers of random 576-byte rows by about a quarter over default-policy loads.
__device__ __forceinline__ void copy16(const uint8_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void copy4(const int32_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dword %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}
// s_waitcnt vmcnt(n) for a wave-uniform n in [0, 15].
__device__ __forceinline__ void wait_vmem(int n) {
    switch (n) {
#define GQA_WAIT_CASE(k) \
    case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
        GQA_WAIT_CASE(0) GQA_WAIT_CASE(1) GQA_WAIT_CASE(2) GQA_WAIT_CASE(3) GQA_WAIT_CASE(4)
        GQA_WAIT_CASE(5) GQA_WAIT_CASE(6) GQA_WAIT_CASE(7) GQA_WAIT_CASE(8) GQA_WAIT_CASE(9)
        GQA_WAIT_CASE(10) GQA_WAIT_CASE(11) GQA_WAIT_CASE(12) GQA_WAIT_CASE(13) GQA_WAIT_CASE(14)
#undef GQA_WAIT_CASE
        default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}

// Loads 8 bf16 query values at d (< DQK) of one row: the latent part from q, the rope part from
// q_pe.  8-element pieces never straddle the boundary (it is a multiple of 8).
template <int DLAT>
__device__ __forceinline__ u32x4 load_q8(const uint16_t *ql, const uint16_t *qp, int d) {
    return d < DLAT ? *reinterpret_cast<const u32x4 *>(ql + d)
                    : *reinterpret_cast<const u32x4 *>(qp + (d - DLAT));
}

// x (|x| < 448) -> (hi, lo) e4m3 quads: hi = nearest, lo = nearest to the remainder.
__device__ __forceinline__ void split_fp8x4(float x0, float x1, float x2, float x3, int &hi, int &lo) {
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
    const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01.x, x1 - h01.y, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23.x, x3 - h23.y, lo, true);
}

// Max / sum of the values of lanes l and l ^ 32, identical in both: v_permlane32_swap hands back
// the values of lanes l & 31 and (l & 31) + 32.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int DQK, int DV, bool DIRECT>
__global__ void __launch_bounds__(kThreads, 1) mla_split_kernel(const MlaSplitArgs a) {
    using T = MlaLayout<DQK>;
    constexpr int DLAT = DQK - 64;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T::kLdsBytes];

    const int logical = xcd_logical_block(blockIdx.x, a.total_ctas);
    if (logical < 0) return;
    const int rblk = logical % a.row_blocks;
    const int rest = logical / a.row_blocks;
    const int part = rest % a.np;
    const int b = rest / a.np;

    // Keys of this partition: ceil(S / np) rounded up to block_k, the last ones possibly empty;
    // no row of the block sees past the block's latest draft token.
    const int S = a.seq_lens[b];
    const int base = a.kv_indptr[b];
    const int chunk = ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int row0 = rblk * kBM;
    const int nrows = min(kBM, a.rows_per_req - row0);
    const int k1 = min(max(0, S - a.q_len + (row0 + nrows - 1) / a.H + 1), k0 + chunk);
    const int kfull = min(k1, max(0, S - a.q_len + row0 / a.H + 1));  // keys every row sees
    const int ntiles = k1 > k0 ? (k1 - k0 + kBK - 1) / kBK : 0;
    // Tiles whose keys every row of the block sees need no mask.
    const int n_full = min(ntiles, max(0, (kfull - k0) / kBK));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;   // 32x32 operand / result coordinates
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    uint8_t *const P = lds + T::kPOff;
    uint8_t *const ML = lds + T::kMlOff;

    if (wave < 4) {
        // ================================ score wave ================================
        const int rb = wave & 1, kb = wave >> 1;
        const int rl = 32 * rb + n;             // row within the block
        const bool row_ok = rl < nrows;
        int p_end;                              // keys visible to this row
        float c_row;                            // base-2 score per unit of the raw product
        i32x8 qhi[T::kSteps], qlo[T::kSteps];
        {
            const int r = row0 + rl;
            const int t = row_ok ? r / a.H : 0;
            const int hh = row_ok ? r - t * a.H : 0;
            p_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;
            const int64_t tok = int64_t(b) * a.q_len + t;
            const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(hh) * a.q_st_head;
            const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(hh) * a.qpe_st_head;
            // lane (n, h) of step s holds d = 64 s + 16 h + e (operand bytes 0-15) and
            // d = 64 s + 32 + 16 h + e (bytes 16-31), e = 0..15; piece p of 8 values starts at
            // 64 s + 32 (p >> 1) + 16 h + 8 (p & 1)
            float mx = 0.f;
            if (row_ok) {
#pragma unroll
                for (int s = 0; s < T::kSteps; ++s)
#pragma unroll
                    for (int pc = 0; pc < 4; ++pc) {
                        const u32x4 w4 = load_q8<DLAT>(ql, qp, 64 * s + 32 * (pc >> 1) + 16 * h + 8 * (pc & 1));
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            mx = fmaxf(mx, fmaxf(fabsf(bf16_lo(w4[w])), fabsf(bf16_hi(w4[w]))));
                    }
            }
            mx = pair_max(mx);
            int ex = 0;
            if (mx > 0.f) frexpf(mx, &ex);            // mx = f * 2^ex, f in [0.5, 1)
            const float qs = ldexpf(1.f, 8 - ex);     // row maximum scaled into [128, 256)
            c_row = a.score_scale * ldexpf(1.f, ex - 8);
            // second pass over the same (cached) values: the first pass's registers are free
            asm volatile("" ::: "memory");
#pragma unroll
            for (int s = 0; s < T::kSteps; ++s)
#pragma unroll
                for (int pc = 0; pc < 4; ++pc) {
                    const u32x4 w4 = row_ok ? load_q8<DLAT>(ql, qp, 64 * s + 32 * (pc >> 1) + 16 * h + 8 * (pc & 1))
                                            : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
                    for (int w = 0; w < 4; w += 2) {
                        int hi, lo;
                        split_fp8x4(bf16_lo(w4[w]) * qs, bf16_hi(w4[w]) * qs,
                                    bf16_lo(w4[w + 1]) * qs, bf16_hi(w4[w + 1]) * qs, hi, lo);
                        qhi[s][2 * pc + w / 2] = hi;
                        qlo[s][2 * pc + w / 2] = lo;
                    }
                }
        }

        // Loop-invariant LDS offsets of this lane's K operand (key at tile position 32 kb + n):
        // bytes 0-15 are chunk 4 (s & 1) + h of line s / 2, bytes 16-31 chunk 4 (s & 1) + 2 + h.
        const int pos = 32 * kb + n;
        const int k_off00 = line_off(0, pos, h), k_off01 = line_off(0, pos, 2 + h);
        const int k_off10 = line_off(0, pos, 4 + h), k_off11 = line_off(0, pos, 6 + h);
        const int k_tail0 = tail_off(pos, h), k_tail1 = tail_off(pos, 2 + h);
        // P words of this lane: keys 32 kb + 8 q + 4 h .. + 3 of row rl (q = 0..3), at 16-byte
        // chunk 2 kb + q / 2 of the 64-byte row, chunks swizzled by the row
        const int p_sw = (rl >> 2) & 3;
        int p_wr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
            p_wr[q] = rl * 64 + (((2 * kb + (q >> 1)) ^ p_sw) << 4) + 8 * (q & 1) + 4 * h;
        // Score v (= 4 q + r) of this lane is key 8 q + 4 h + r of the block, tile position
        // 32 kb + 8 q + 4 h + r, slot-list index 32 h + 8 r + 4 kb + q (key_of_pos).
        const int kidx_base = 32 * h + 4 * kb;

        for (int t = 0; t < ntiles; ++t) {
            if (t == 0) __syncthreads();   // tile 0 landed (the value waves' prologue)
            const uint8_t *tb = lds + (t % kSlots) * T::kSlotBytes;
            f32x16 sacc;
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
            for (int s = 0; s < T::kSteps; ++s) {
                u32x4 lo16, hi16;
                if (T::kTail && s == T::kSteps - 1) {
                    lo16 = *reinterpret_cast<const u32x4 *>(tb + k_tail0);
                    hi16 = *reinterpret_cast<const u32x4 *>(tb + k_tail1);
                } else {
                    const int lb = (s >> 1) * 8192;
                    lo16 = *reinterpret_cast<const u32x4 *>(tb + lb + ((s & 1) ? k_off10 : k_off00));
                    hi16 = *reinterpret_cast<const u32x4 *>(tb + lb + ((s & 1) ? k_off11 : k_off01));
                }
                const i32x8 kraw = i32x8{int(lo16.x), int(lo16.y), int(lo16.z), int(lo16.w),
                                         int(hi16.x), int(hi16.y), int(hi16.z), int(hi16.w)};
                sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kraw, qhi[s], sacc, 0, 0, 0, 127, 0, 127);
                sacc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kraw, qlo[s], sacc, 0, 0, 0, 127, 0, 127);
            }

            // Softmax of this 32-key block in base 2 with an integer maximum m:
            // p * 2^8 = 2^(score - m + 8) in (0, 256].
            if (t >= n_full) {
                const int thr = p_end - k0 - t * kBK - kidx_base;   // visible: index - base < thr
#pragma unroll
                for (int vv = 0; vv < 16; ++vv)
                    if (8 * (vv & 3) + (vv >> 2) >= thr) sacc[vv] = kNegInf;
            }
            float mx = sacc[0];
#pragma unroll
            for (int vv = 1; vv < 16; ++vv) mx = fmaxf(mx, sacc[vv]);
            mx = pair_max(mx);
            const int m = mx == kNegInf ? kNoMax : int(ceilf(mx * c_row));
            const float bias = float(8 - m);
            float p[16];
            float esum = 0.f, qsum = 0.f;
#pragma unroll
            for (int vv = 0; vv < 16; ++vv) {
                p[vv] = fast_exp2(fmaf(sacc[vv], c_row, bias));
                esum += p[vv];
            }
            int whi[4], wlo[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                split_fp8x4(p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3], whi[q], wlo[q]);
                const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(whi[q], false);
                const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(whi[q], true);
                const f32x2 l01 = __builtin_amdgcn_cvt_pk_f32_fp8(wlo[q], false);
                const f32x2 l23 = __builtin_amdgcn_cvt_pk_f32_fp8(wlo[q], true);
                qsum += ((h01.x + l01.x) + (h01.y + l01.y)) + ((h23.x + l23.x) + (h23.y + l23.y));
            }
            esum = pair_sum(esum);
            qsum = pair_sum(qsum);
            uint8_t *pb = P + (t & 1) * 8192;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                *reinterpret_cast<int *>(pb + p_wr[q]) = whi[q];
                *reinterpret_cast<int *>(pb + 4096 + p_wr[q]) = wlo[q];
            }
            if (h == 0)
                *reinterpret_cast<i32x4 *>(ML + (t & 1) * 2048 + rl * 32 + kb * 16) =
                    i32x4{m, __float_as_int(qsum), __float_as_int(esum), 0};
            __syncthreads();   // P(t) published; tile t + 1 landed
        }
        return;
    }

    // ================================ value wave ================================
    const int v = wave - 4;   // output columns 128 v .. 128 v + 127 = line v of the rows
    // ---- copies.  Instruction i writes tile positions 8 i .. 8 i + 7 of line v: lane L carries
    // slot-list key 8 (L >> 3) + i at position 8 i + (L >> 3), chunk position L & 7, i.e. global
    // chunk (L & 7) ^ swz_line(position).  The tail copy writes positions 16 v .. 16 v + 15.
    const int jgrp = lane >> 3;
    const int tail_pos = 16 * v + (lane >> 2);
    const int tail_chunk = 512 + 16 * ((lane & 3) ^ swz_tail(tail_pos));
    const int tail_key = key_of_pos(tail_pos);
    const int32_t *const ibase = a.kv_indices + base;
    const uint64_t kv_stride = uint64_t(a.kv_stride);
    const uint8_t *const kv_line = a.kv + 128 * v;
    const uint32_t id_lds = lds_addr + T::kIdOff + v * (kIdSlots * 256);
    const int32_t *const id_ring = reinterpret_cast<const int32_t *>(lds + T::kIdOff + v * (kIdSlots * 256));

    auto issue_ids = [&](int tile) {
        if (tile < ntiles)
            copy4(ibase + min(k0 + tile * kBK + lane, k1 - 1), id_lds + (tile % kIdSlots) * 256);
    };
    auto issue_rows = [&](int tile) {
        if (tile >= ntiles) return;
        const int32_t *ids = id_ring + (tile % kIdSlots) * 64;
        const u32x4 ia = *reinterpret_cast<const u32x4 *>(ids + 8 * jgrp);
        const u32x4 ib = *reinterpret_cast<const u32x4 *>(ids + 8 * jgrp + 4);
        const uint32_t slot = lds_addr + (tile % kSlots) * T::kSlotBytes;
        const uint32_t idv[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gc = (lane & 7) ^ (((i & 1) << 2) | (jgrp >> 1));
            copy16(kv_line + uint64_t(idv[i]) * kv_stride + 16 * gc, slot + v * 8192 + 1024 * i);
        }
        if (T::kTail) {
            const uint32_t idt = uint32_t(ids[tail_key]);
            copy16(a.kv + uint64_t(idt) * kv_stride + tail_chunk, slot + 32768 + 1024 * v);
        }
    };
    // Issue order: ids(0), ids(1), then rows(j), ids(j + 2) for j = 0, 1, 2, ...; operations for
    // tiles >= ntiles are skipped.  Copies retire in issue order.
    constexpr int NC = T::kCopies;
    auto cnt_rows = [&](int j) { return j >= 0 && j < ntiles ? NC : 0; };
    auto cnt_ids = [&](int j) { return j >= 0 && j < ntiles ? 1 : 0; };
    // before rows(j): ids(j) landed; issued after it: rows(j - 1), ids(j + 1)
    auto wait_ids = [&](int j) { wait_vmem(cnt_rows(j - 1) + cnt_ids(j + 1)); };
    // rows(j) landed; issued after it: ids(j + 2), rows(j + 1), ids(j + 3)
    auto wait_rows = [&](int j) { wait_vmem(cnt_ids(j + 2) + cnt_rows(j + 1) + cnt_ids(j + 3)); };

    // ---- PV operands.  V^T (A operand) of column block cb: lane (m, h) holds keys 16 h + 0..15
    // (bytes 0-15) and 32 + 16 h + 0..15 (bytes 16-31) of column m; a transposed read hands a
    // 16-lane group 8 keys of 16 columns: lane s = 2 k + hh points at key k of the read, bytes
    // 8 hh.. of the chunk (cb for lanes 0-15 of each half-wave, cb ^ 4 for lanes 16-31).
    const int kk = (lane & 15) >> 1, hh = lane & 1, half = (lane >> 4) & 1;
    int v_off[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v_off[cb][r] = line_off(v, 16 * h + 8 * (r & 1) + 32 * (r >> 1) + kk, half ? (cb ^ 4) : cb) + 8 * hh;
    //   P^T (B operand) of row 32 rb + n: keys 16 h .. (chunk h) and 32 + 16 h .. (chunk 2 + h)
    int p_rd[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = 32 * rb + n, sw = (row >> 2) & 3;
        p_rd[rb][0] = row * 64 + ((h ^ sw) << 4);
        p_rd[rb][1] = row * 64 + (((2 + h) ^ sw) << 4);
    }

    int mc[2] = {kNoMax, kNoMax};   // running integer maxima of rows n and 32 + n
    float lq[2] = {0.f, 0.f};       // running sums of the applied (quantized) weights
    float le[2] = {0.f, 0.f};       // running sums of 2^(score - mc)
    f32x16 oacc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[rb][cb][i] = 0.f;

    // PV of tile t: running maxima and sums, the rescale when a maximum moved, then 16 MFMAs.
    auto pv = [&](int t) {
        const uint8_t *pbuf = P + (t & 1) * 8192;
        const uint8_t *mlb = ML + (t & 1) * 2048;
        int sc[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const i32x4 m0 = *reinterpret_cast<const i32x4 *>(mlb + (32 * rb + n) * 32);
            const i32x4 m1 = *reinterpret_cast<const i32x4 *>(mlb + (32 * rb + n) * 32 + 16);
            const int m_new = max(mc[rb], max(m0.x, m1.x));
            const float alpha = ldexpf(1.f, mc[rb] - m_new);
            lq[rb] = lq[rb] * alpha + ldexpf(__int_as_float(m0.y), m0.x - m_new - 8) +
                     ldexpf(__int_as_float(m1.y), m1.x - m_new - 8);
            le[rb] = le[rb] * alpha + ldexpf(__int_as_float(m0.z), m0.x - m_new - 8) +
                     ldexpf(__int_as_float(m1.z), m1.x - m_new - 8);
            mc[rb] = m_new;
            sc[rb] = max(0, 127 - 8 + (h ? m1.x : m0.x) - m_new);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int cb = 0; cb < 4; ++cb) oacc[rb][cb] *= alpha;
            }
        }
        i32x8 ph[2], pl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(pbuf + p_rd[rb][0]);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(pbuf + p_rd[rb][1]);
            const u32x4 b0 = *reinterpret_cast<const u32x4 *>(pbuf + 4096 + p_rd[rb][0]);
            const u32x4 b1 = *reinterpret_cast<const u32x4 *>(pbuf + 4096 + p_rd[rb][1]);
            ph[rb] = i32x8{int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
            pl[rb] = i32x8{int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
        }
        const uint8_t *tb = lds + (t % kSlots) * T::kSlotBytes;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            int2v raw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                raw[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(tb + v_off[cb][r]));
            const i32x8 vt = i32x8{raw[0].x, raw[0].y, raw[1].x, raw[1].y,
                                   raw[2].x, raw[2].y, raw[3].x, raw[3].y};
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                oacc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    vt, ph[rb], oacc[rb][cb], 0, 0, 0, 127, 0, sc[rb]);
                oacc[rb][cb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    vt, pl[rb], oacc[rb][cb], 0, 0, 0, 127, 0, sc[rb]);
            }
        }
    };

    if (ntiles > 0) {
        issue_ids(0);
        issue_ids(1);
        wait_ids(0);
        issue_rows(0);
        issue_ids(2);
        wait_ids(1);
        issue_rows(1);
        issue_ids(3);
        wait_rows(0);
        __syncthreads();   // tile 0 landed
        for (int t = 0; t < ntiles; ++t) {
            if (t > 0) pv(t - 1);
            // slot (t + 2) % 3 held tile t - 1: every read of it is done (the score waves' in the
            // previous step, this wave's own line just above)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            wait_ids(t + 2);
            issue_rows(t + 2);
            issue_ids(t + 4);
            if (t + 1 < ntiles) wait_rows(t + 1);
            __syncthreads();   // P(t) published; tile t + 1 landed
        }
        pv(ntiles - 1);
    }

    // ---- epilogue: lane (n, h) of block cb holds columns m = 8 q + 4 h + 0..3 of row 32 rb + n;
    // m < 16 lie in chunk cb of line v, the others in chunk cb ^ 4.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int rl = 32 * rb + n;
        if (rl >= nrows) continue;
        const int64_t row = int64_t(b) * a.rows_per_req + row0 + rl;
        const float inv = lq[rb] > 0.f ? a.out_scale / lq[rb] : 0.f;
        const float lse2 = le[rb] > 0.f ? float(mc[rb]) + __log2f(le[rb]) : kNegInf;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = 128 * v + 16 * (q < 2 ? cb : (cb ^ 4)) + 8 * (q & 1) + 4 * h;
                if (col >= DV) continue;
                const float v0 = oacc[rb][cb][4 * q] * inv, v1 = oacc[rb][cb][4 * q + 1] * inv;
                const float v2 = oacc[rb][cb][4 * q + 2] * inv, v3 = oacc[rb][cb][4 * q + 3] * inv;
                if (DIRECT) {
                    *reinterpret_cast<uint2 *>(a.out + row * DV + col) =
                        make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                } else {
                    *reinterpret_cast<f32x4 *>(a.part_o + (row * a.np + part) * DV + col) =
                        f32x4{v0, v1, v2, v3};
                }
            }
        if (v == 0 && h == 0) {
            if (DIRECT) {
                if (a.lse2_out) a.lse2_out[row] = lse2;
            } else {
                a.part_lse2[row * a.np + part] = lse2;
            }
        }
    }
}

template <int DQK, int DV>
hipError_t launch_shape(const MlaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(kThreads);
    if (direct)
        hipLaunchKernelGGL((mla_split_kernel<DQK, DV, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mla_split_kernel<DQK, DV, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

int mla_rows_per_cta() { return kBM; }

hipError_t launch_mla_split(const MlaSplitArgs &a, int d_qk, int d_v, bool direct, hipStream_t s) {
    if (a.block_k != 32 && a.block_k != 64) return hipErrorInvalidValue;
    if (d_qk == 576 && d_v == 512) return launch_shape<576, 512>(a, direct, s);
    if (d_qk == 512 && d_v == 448) return launch_shape<512, 448>(a, direct, s);
    return hipErrorInvalidValue;
}

}  // namespace gqa
