// mla_split.hip -- split kernel of absorbed MLA decode for gfx950.
//
// What it computes (moonmath-amd README, "MLA decode"; Modular MAX planner page, MLA-style
// bullet): every key row of the pool is one fused fp8 e4m3 row that serves as K (all DQK bytes)
// and as V (its first DV bytes), dequantized with one per-tensor kv_scale.  A CTA owns up to 64
// query rows of one request and walks one partition of that request's keys, writing the
// partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Layout of the work (512 threads = 8 waves, one CTA per CU, two waves per SIMD):
//   - Keys arrive in tiles of 64.  Each tile is copied straight from HBM into LDS with
//     global_load_lds_dwordx4 (no register staging), three tiles ahead of the compute, into a
//     ring of four LDS tile buffers.  The copies are issued from inline assembly and waited for
//     with explicit vmcnt counts: the compiler cannot tell which LDS reads a direct copy feeds,
//     and would otherwise drain every copy in flight before each LDS read.
//   - QK^T: wave w computes the scores of key block kb = w % 2 (32 keys) for query-row quarter
//     rq = w / 2 (16 rows) over the whole row width, on the block-scaled fp8 MFMA
//     v_mfma_scale_f32_16x16x128_f8f6f4 with unit scales (the 64-wide rope tail of 576-byte rows
//     on v_mfma_f32_16x16x32_fp8_fp8).  K is used as stored.  A bf16 query row, scaled by a power
//     of two so its largest element lies in [128, 256), is the exact sum of two e4m3 vectors (hi =
//     nearest, lo = remainder) except below e4m3's subnormal step; each product runs twice.
//   - Softmax: each wave reduces its own 16 rows x 32 keys.  The running maximum is kept as an
//     integer (the ceiling of the base-2 score), so probabilities produced by different waves, or
//     in different tiles, differ by exact powers of two.  Probabilities are written to LDS as fp8
//     hi/lo pairs of p * 2^8 (p <= 1), together with each (row, key block) maximum and two sums:
//     of the quantized probabilities (the weights PV applies, which normalize the output) and of
//     the exact ones (which give the log-sum-exp).
//   - PV: wave w owns output columns 32w..32w+31 and 32(w+8).. for all 64 rows, on the 32x32x64
//     block-scaled fp8 MFMA.  V^T is read from the fp8 tile with ds_read_b64_tr_b8 (no
//     conversion); P^T comes from LDS, and the power of two that aligns each 32-key block with
//     the row's running maximum is the MFMA's per-lane B scale.
//
// LDS tile layout: a key row is cut into 128-byte lines (eight 16-byte chunks; the 64-byte rope
// tail of 576-byte rows is a half line).  Line j < 4 of all 64 keys fills 8 KiB at j * 8192, key k
// at k * 128, its chunks permuted by an XOR with swz8(k); the half line fills 4 KiB at 32768, key
// k at k * 64, chunks permuted with swz4(k).  A direct copy writes 64 consecutive 16-byte slots,
// so one copy instruction moves whole lines (8 keys x 8 chunks, or 16 keys x 4 chunks of the half
// line) and each cache line of a row is fetched once.  The permutations keep the score-operand reads (16
// keys, one chunk pair), the transposed value reads (8 keys x 16 bytes) and the copies free of
// bank conflicts.
#include "device_common.hpp"
#include "kernels.hpp"

#include <type_traits>

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
constexpr int kBufs = 4;           // LDS tile ring
constexpr int kNoMax = -(1 << 20); // integer maximum of a block with no visible key

template <int DQK, int DV>
struct MlaShape {
    static constexpr int kChunks = DQK / 16;              // 16-byte chunks per key row
    static constexpr int kTileBytes = kBK * DQK;
    static constexpr int kRopeSteps = (DQK - 512) / 32;   // 32-wide fp8 steps past byte 512
    static constexpr int kDvBlocks = DV / 32;             // 32-column output blocks
    static constexpr int kPOff = kBufs * kTileBytes;      // P hi [64 rows][64 keys], then P lo
    // per row: m0, m1 (int); quantized sums q0, q1; exact sums e0, e1 (float); two pad words
    static constexpr int kMlOff = kPOff + 2 * kBM * kBK;
    static constexpr int kIdxOff = kMlOff + kBM * 32;     // per wave, two slots of 64 slot ids
    static constexpr int kLdsBytes = kIdxOff + 8 * 2 * 256;
    static_assert(DQK == 576 || DQK == 512, "row width");
    static_assert(DV % 32 == 0 && DV <= 512, "value width");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

__device__ __forceinline__ int swz8(int key) { return (((key >> 1) & 3) << 1) | ((key >> 3) & 1); }
__device__ __forceinline__ int swz4(int key) { return (key >> 2) & 3; }
// Byte offset of 16-byte chunk c of tile key `key` (see the layout note above).
__device__ __forceinline__ int tpos(int c, int key) {
    return c < 32 ? (c >> 3) * 8192 + key * 128 + (((c & 7) ^ swz8(key)) << 4)
                  : 32768 + key * 64 + (((c & 3) ^ swz4(key)) << 4);
}

// Direct HBM -> LDS copy of 16 bytes per lane: lane L's bytes land at m0 + OFF + 16 L; the
// immediate offset applies to the global address too.
template <int OFF>
__device__ __forceinline__ void copy16(const uint8_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, off offset:%1" ::"v"(g), "i"(OFF), "{m0}"(m0) : "memory");
}
// Same, 4 bytes per lane (lane L -> m0 + 4 L).
__device__ __forceinline__ void copy4(const int32_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(m0) : "memory");
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

// Max / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (one per 16-lane row), identical in all
// four: v_permlane32_swap and v_permlane16_swap exchange rows without going through LDS.
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

// x (|x| < 448) -> (hi, lo) e4m3 quads: hi = nearest, lo = nearest to the remainder.
__device__ __forceinline__ void split_fp8x4(float x0, float x1, float x2, float x3, int &hi, int &lo) {
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
    const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
    const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01.x, x1 - h01.y, 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23.x, x3 - h23.y, lo, true);
}

template <int DQK, int DV, bool DIRECT>
__global__ void __launch_bounds__(kThreads, 1) mla_split_kernel(const MlaSplitArgs a) {
    using T = MlaShape<DQK, DV>;
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

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb = wave & 1, rq = wave >> 1;
    const int n16 = lane & 15, g = lane >> 4;   // 16x16 operand / result coordinates
    const int n32 = lane & 31, h = lane >> 5;   // 32x32 operand / result coordinates

    // ---- producer row (QK^T and softmax): row 16 rq + n16 of the block
    const int prow = 16 * rq + n16;
    const bool prow_ok = prow < nrows;
    int p_end;   // keys visible to this row
    float c_row; // base-2 score per unit of the raw product
    i32x8 qhi[4], qlo[4];
    long qrh[T::kRopeSteps > 0 ? T::kRopeSteps : 1], qrl[T::kRopeSteps > 0 ? T::kRopeSteps : 1];
    {
        const int r = row0 + prow;
        const int t = prow_ok ? r / a.H : 0;
        const int hh = prow_ok ? r - t * a.H : 0;
        p_end = prow_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;
        const int64_t tok = int64_t(b) * a.q_len + t;
        const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(hh) * a.q_st_head;
        const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(hh) * a.qpe_st_head;
        // lane (n16, g) holds d = 128 s + 32 g + e of step s, and d = 512 + 32 st + 8 g + e of
        // rope step st
        float qv[4][32];
        float qr[T::kRopeSteps > 0 ? T::kRopeSteps : 1][8];
        float mx = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (prow_ok) v = load_q8<DLAT>(ql, qp, 128 * s + 32 * g + 8 * e);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    qv[s][8 * e + 2 * w] = bf16_lo(v[w]);
                    qv[s][8 * e + 2 * w + 1] = bf16_hi(v[w]);
                    mx = fmaxf(mx, fmaxf(fabsf(qv[s][8 * e + 2 * w]), fabsf(qv[s][8 * e + 2 * w + 1])));
                }
            }
#pragma unroll
        for (int st = 0; st < T::kRopeSteps; ++st) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (prow_ok) v = load_q8<DLAT>(ql, qp, 512 + 32 * st + 8 * g);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                qr[st][2 * w] = bf16_lo(v[w]);
                qr[st][2 * w + 1] = bf16_hi(v[w]);
                mx = fmaxf(mx, fmaxf(fabsf(qr[st][2 * w]), fabsf(qr[st][2 * w + 1])));
            }
        }
        mx = fmaxf(mx, xor_shuffle(mx, 16));
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        int ex = 0;
        if (mx > 0.f) frexpf(mx, &ex);            // mx = f * 2^ex, f in [0.5, 1)
        const float qs = ldexpf(1.f, 8 - ex);     // row maximum scaled into [128, 256)
        c_row = a.score_scale * ldexpf(1.f, ex - 8);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                int hi, lo;
                split_fp8x4(qv[s][4 * w] * qs, qv[s][4 * w + 1] * qs, qv[s][4 * w + 2] * qs,
                            qv[s][4 * w + 3] * qs, hi, lo);
                qhi[s][w] = hi;
                qlo[s][w] = lo;
            }
#pragma unroll
        for (int st = 0; st < T::kRopeSteps; ++st) {
            int h0, l0, h1, l1;
            split_fp8x4(qr[st][0] * qs, qr[st][1] * qs, qr[st][2] * qs, qr[st][3] * qs, h0, l0);
            split_fp8x4(qr[st][4] * qs, qr[st][5] * qs, qr[st][6] * qs, qr[st][7] * qs, h1, l1);
            qrh[st] = long(uint32_t(h0)) | (long(uint32_t(h1)) << 32);
            qrl[st] = long(uint32_t(l0)) | (long(uint32_t(l1)) << 32);
        }
    }

    // ---- consumer state (PV): rows 32 rb + n32, output blocks wave and wave + 8
    constexpr int kMyBlocks = 2;
    const bool has_blk1 = wave + 8 < T::kDvBlocks;
    int mc[2] = {kNoMax, kNoMax};
    float lc[2] = {0.f, 0.f};   // sum of applied (quantized) weights
    float le[2] = {0.f, 0.f};   // exact sum, for the log-sum-exp
    f32x16 oacc[2][kMyBlocks];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < kMyBlocks; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[rb][j][i] = 0.f;

    // ---- tile copies.  Wave w copies lines 0-3 of keys 8w..8w+7 (lane L: key 8w + L/8, chunk
    // L%8 ^ swz8(key) of the line) and, for 576-byte rows and w < 4, the half line of keys
    // 16w..16w+15 (lane L: key 16w + L/4).  It first copies the tile's 64 slot ids (lane L: key L)
    // into its own LDS index slot.
    const int n_copy = 4 + (T::kChunks > 32 && wave < 4 ? 1 : 0);   // copies per tile
    const int key_a = 8 * wave + (lane >> 3), key_b = 16 * (wave & 3) + (lane >> 2);
    const int chunk_a = 16 * ((lane & 7) ^ swz8(key_a));           // byte offset in the line
    const int chunk_b = 512 + 16 * ((lane & 3) ^ swz4(key_b));
    const int32_t *const ibase = a.kv_indices + base;
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    const int32_t *const idx_lds = reinterpret_cast<const int32_t *>(lds + T::kIdxOff) + wave * 128;
    const uint64_t kv_stride = uint64_t(a.kv_stride);

    auto issue_idx = [&](int tile) {
        const int key = min(k0 + tile * kBK + lane, k1 - 1);
        copy4(ibase + key, lds_addr + T::kIdxOff + (wave * 2 + (tile & 1)) * 256);
    };
    auto issue_rows = [&](int tile) {
        const int32_t *ids = idx_lds + (tile & 1) * 64;
        const uint8_t *row = a.kv + uint64_t(uint32_t(ids[key_a])) * kv_stride + chunk_a;
        const uint32_t m0 = lds_addr + (tile & (kBufs - 1)) * T::kTileBytes + wave * 1024;
        // copy u moves line u: LDS + 8 KiB, global + 128 bytes per step
        copy16<0>(row, m0);
        copy16<128>(row, m0 + 8192 - 128);
        copy16<256>(row, m0 + 16384 - 256);
        copy16<384>(row, m0 + 24576 - 384);
        if (n_copy > 4) {
            const uint8_t *row_b = a.kv + uint64_t(uint32_t(ids[key_b])) * kv_stride + chunk_b;
            copy16<0>(row_b, m0 + 32768);
        }
    };
    // Copies retire in issue order.  Per tile j (issue order): slot ids of j + 1, then rows of j.
    // Before the rows of j + 3: the ids of j + 3 landed; after them came rows j + 2 and ids j + 4.
    auto wait_ids = [&](int j) {
        wait_vmem((j + 2 >= 0 && j + 2 < ntiles ? n_copy : 0) + (j + 4 < ntiles ? 1 : 0));
    };
    // Before compute on tile t + 1: its rows landed; after them came ids t + 3, rows t + 2,
    // ids t + 4, rows t + 3.
    auto wait_rows = [&](int t) {
        wait_vmem((t + 3 < ntiles ? 1 + n_copy : 0) + (t + 2 < ntiles ? n_copy : 0) +
                  (t + 4 < ntiles ? 1 : 0));
    };

    uint8_t *const P = lds + T::kPOff;
    uint8_t *const ML = lds + T::kMlOff;

    // Loop-invariant LDS byte offsets of this lane's operands; a tile base and immediates are
    // added per read.
    //   score operand, key 32 kb + 16 sb + n16: chunks 8 s + 2 g and 8 s + 2 g + 1 (line s; sb
    //   adds 16 keys = 2048 bytes)
    const int k_even = tpos(2 * g, 32 * kb + n16);
    const int k_odd = tpos(2 * g + 1, 32 * kb + n16);
    //   rope operand: chunk 32 + 2 st + g / 2, bytes 8 (g % 2).. (sb adds 16 keys = 1024 bytes)
    const int k_rope0 = tpos(32 + (g >> 1), 32 * kb + n16) + 8 * (g & 1);
    const int k_rope1 = tpos(34 + (g >> 1), 32 * kb + n16) + 8 * (g & 1);
    //   V^T operand: lane (m = dv column, h) holds keys 16h + 0..15 (bytes 0-15) and 32 + 16h +
    //   0..15 (bytes 16-31).  A transposed read gives 8 keys of one column: lane s = 2k + hh of a
    //   16-lane group points at key k of the read (keys 32 (r / 2) + 16 h + 8 (r % 2) + k of
    //   chunk 2 (wave + 8 j) + half), column bytes 8hh..8hh+7.  32 keys = 4096 bytes; j adds two
    //   lines.
    const int kk = (lane & 15) >> 1, hh = lane & 1, half = (lane >> 4) & 1;
    const int v_base0 = tpos(2 * wave + half, 16 * h + kk) + 8 * hh;
    const int v_base1 = tpos(2 * wave + half, 16 * h + 8 + kk) + 8 * hh;
    //   P^T operand of row 32 rb + n32: keys 16h.. and 32 + 16h.. (16-byte chunks, swizzled by row)
    const int p_sw = (n32 >> 2) & 3;
    const int p_rd0 = n32 * 64 + ((h ^ p_sw) << 4), p_rd1 = n32 * 64 + (((2 + h) ^ p_sw) << 4);
    //   this producer lane's words: keys 32 kb + 16 sb + 4 g .. + 3 of row prow
    const int pw_sw = (prow >> 2) & 3;
    const int p_wr0 = prow * 64 + (((2 * kb) ^ pw_sw) << 4) + 4 * g;
    const int p_wr1 = prow * 64 + (((2 * kb + 1) ^ pw_sw) << 4) + 4 * g;
    // the last output block of a 448-wide value exists for waves 0-5 only; the others read a
    // valid (unused) chunk and drop the result
    const int v_blk1 = has_blk1 ? 16384 : 0;
    // Tiles whose keys every row of the block sees need no mask.
    const int n_full = min(ntiles, max(0, (kfull - k0) / kBK));

    auto tile_ptr = [&](int t) -> const uint8_t * { return lds + (t & (kBufs - 1)) * T::kTileBytes; };

    auto qk = [&](const uint8_t *tb, f32x4 (&sacc)[2]) {
        sacc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
        sacc[1] = sacc[0];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const u32x4 lo16 = *reinterpret_cast<const u32x4 *>(tb + k_even + 8192 * s + 2048 * sb);
                const u32x4 hi16 = *reinterpret_cast<const u32x4 *>(tb + k_odd + 8192 * s + 2048 * sb);
                const i32x8 kraw = i32x8{int(lo16.x), int(lo16.y), int(lo16.z), int(lo16.w),
                                         int(hi16.x), int(hi16.y), int(hi16.z), int(hi16.w)};
                sacc[sb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    kraw, qhi[s], sacc[sb], 0, 0, 0, 127, 0, 127);
                sacc[sb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    kraw, qlo[s], sacc[sb], 0, 0, 0, 127, 0, 127);
            }
#pragma unroll
        for (int st = 0; st < T::kRopeSteps; ++st)
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {
                const long kr = *reinterpret_cast<const long *>(tb + (st ? k_rope1 : k_rope0) + 1024 * sb);
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kr, qrh[st], sacc[sb], 0, 0, 0);
                sacc[sb] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(kr, qrl[st], sacc[sb], 0, 0, 0);
            }
    };

    // PV bookkeeping for the probabilities now in LDS: new running maxima and sums, the rescale
    // of the accumulators when a maximum moved, and each lane's B scale.
    auto pv_prep = [&](int (&sc)[2]) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const i32x4 ml = *reinterpret_cast<const i32x4 *>(ML + n32 * 32 + 1024 * rb);
            const f32x2 ex = *reinterpret_cast<const f32x2 *>(ML + n32 * 32 + 1024 * rb + 16);
            const int m_new = max(mc[rb], max(ml.x, ml.y));
            const float alpha = ldexpf(1.f, mc[rb] - m_new);
            lc[rb] = lc[rb] * alpha + ldexpf(__int_as_float(ml.z), ml.x - m_new - 8) +
                     ldexpf(__int_as_float(ml.w), ml.y - m_new - 8);
            le[rb] = le[rb] * alpha + ldexpf(ex.x, ml.x - m_new - 8) + ldexpf(ex.y, ml.y - m_new - 8);
            mc[rb] = m_new;
            sc[rb] = max(0, 127 - 8 + (h ? ml.y : ml.x) - m_new);
            if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                for (int j = 0; j < kMyBlocks; ++j) oacc[rb][j] *= alpha;
            }
        }
    };

    auto pv_mma = [&](const uint8_t *tb, const int (&sc)[2]) {
        i32x8 ph[2], pl[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const u32x4 a0 = *reinterpret_cast<const u32x4 *>(P + p_rd0 + 2048 * rb);
            const u32x4 a1 = *reinterpret_cast<const u32x4 *>(P + p_rd1 + 2048 * rb);
            const u32x4 b0 = *reinterpret_cast<const u32x4 *>(P + 4096 + p_rd0 + 2048 * rb);
            const u32x4 b1 = *reinterpret_cast<const u32x4 *>(P + 4096 + p_rd1 + 2048 * rb);
            ph[rb] = i32x8{int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
            pl[rb] = i32x8{int(b0.x), int(b0.y), int(b0.z), int(b0.w), int(b1.x), int(b1.y), int(b1.z), int(b1.w)};
        }
#pragma unroll
        for (int j = 0; j < kMyBlocks; ++j) {
            const uint8_t *vb = tb + (j ? v_blk1 : 0);
            int2v raw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
                raw[r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(vb + ((r & 1) ? v_base1 : v_base0) + 4096 * (r >> 1)));
            const i32x8 vt = i32x8{raw[0].x, raw[0].y, raw[1].x, raw[1].y,
                                   raw[2].x, raw[2].y, raw[3].x, raw[3].y};
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                oacc[rb][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    vt, ph[rb], oacc[rb][j], 0, 0, 0, 127, 0, sc[rb]);
                oacc[rb][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    vt, pl[rb], oacc[rb][j], 0, 0, 0, 127, 0, sc[rb]);
            }
        }
    };

    // Softmax of this wave's block in base 2 with an integer maximum m:
    // p * 2^8 = 2^(score - m + 8) in (0, 256].  Returns the hi/lo words, m and both row sums.
    struct Probs {
        int whi[2], wlo[2];
        int m;
        float lsum, esum;
    };
    auto softmax = [&](int t, f32x4 (&sacc)[2], auto masked) -> Probs {
        if constexpr (decltype(masked)::value) {
            const int kt = k0 + t * kBK + 32 * kb;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (kt + 16 * sb + 4 * g + i >= p_end) sacc[sb][i] = kNegInf;
        }
        Probs r;
        float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                         fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
        mx = rows4_max(mx);
        r.m = mx == kNegInf ? kNoMax : int(ceilf(mx * c_row));
        const float bias = float(8 - r.m);
        // The row sum adds the probabilities as quantized (hi + lo), the weights PV applies: a
        // dominant key then carries no quantization error into the normalized output.
        float lsum = 0.f, esum = 0.f;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(fmaf(sacc[sb][i], c_row, bias));
                esum += p[i];
            }
            split_fp8x4(p[0], p[1], p[2], p[3], r.whi[sb], r.wlo[sb]);
            const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(r.whi[sb], false);
            const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(r.whi[sb], true);
            const f32x2 l01 = __builtin_amdgcn_cvt_pk_f32_fp8(r.wlo[sb], false);
            const f32x2 l23 = __builtin_amdgcn_cvt_pk_f32_fp8(r.wlo[sb], true);
            lsum += ((h01.x + l01.x) + (h01.y + l01.y)) + ((h23.x + l23.x) + (h23.y + l23.y));
        }
        r.lsum = rows4_sum(lsum);
        r.esum = rows4_sum(esum);
        return r;
    };

    auto publish = [&](const Probs &pr) {
        *reinterpret_cast<int *>(P + p_wr0) = pr.whi[0];
        *reinterpret_cast<int *>(P + p_wr1) = pr.whi[1];
        *reinterpret_cast<int *>(P + 4096 + p_wr0) = pr.wlo[0];
        *reinterpret_cast<int *>(P + 4096 + p_wr1) = pr.wlo[1];
        if (g == 0) {
            *reinterpret_cast<int *>(ML + prow * 32 + 4 * kb) = pr.m;
            *reinterpret_cast<float *>(ML + prow * 32 + 8 + 4 * kb) = pr.lsum;
            *reinterpret_cast<float *>(ML + prow * 32 + 16 + 4 * kb) = pr.esum;
        }
    };

    // Copies for later tiles, then the wait for tile t + 1 (constant counts in steady state).
    auto advance = [&](int t) {
        if (t + 4 < ntiles) {
            issue_idx(t + 4);
            if (n_copy > 4) {
                asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
                issue_rows(t + 3);
                asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
            } else {
                asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
                issue_rows(t + 3);
                asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
            }
        } else {
            if (t + 3 < ntiles) {
                wait_ids(t);
                issue_rows(t + 3);
            }
            if (t + 1 < ntiles) wait_rows(t);
        }
    };

    // One tile: scores of t, PV of t - 1 and the softmax of t in one straight-line block (so the
    // MFMAs of one overlap the VALU work of the other), then the exchange of P(t).
    auto step = [&](int t, auto masked, auto first) {
        int sc[2] = {0, 0};
        f32x4 sacc[2];
        qk(tile_ptr(t), sacc);
        // scores: each step's four operand reads go out one step ahead of its four MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int s = 0; s < 4 + T::kRopeSteps / 2; ++s) {
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the PV bookkeeping's VALU work runs while the score MFMAs drain
        if constexpr (!decltype(first)::value) pv_prep(sc);
        if constexpr (!decltype(first)::value) pv_mma(tile_ptr(t - 1), sc);
        const Probs pr = softmax(t, sacc, masked);
        if constexpr (!decltype(first)::value) {
            // PV's operand reads first, then its eight MFMAs spread through the softmax VALU work
            __builtin_amdgcn_sched_group_barrier(0x100, 16, 1);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
                __builtin_amdgcn_sched_group_barrier(0x002, 12, 1);
            }
        }
        if constexpr (!decltype(first)::value) {
            // an empty use of the accumulators here keeps the PV MFMAs in this block (the
            // compiler would otherwise sink them past the barrier, away from the softmax)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                for (int j = 0; j < kMyBlocks; ++j) asm volatile("" : "+v"(oacc[rb][j]));
        }
        __builtin_amdgcn_sched_barrier(0);   // keep the softmax ahead of the barrier
        if constexpr (!decltype(first)::value)
            __syncthreads();   // every wave is done with PV(t - 1): P, ML and buffer (t - 1) % 4 free
        publish(pr);
        advance(t);
        __syncthreads();       // P(t) and tile t + 1 visible to every wave
    };

    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    if (ntiles > 0) {
        issue_idx(0);
#pragma unroll
        for (int j = -3; j < 0; ++j) {
            if (j + 4 < ntiles) issue_idx(j + 4);
            if (j + 3 < ntiles) {
                wait_ids(j);
                issue_rows(j + 3);
            }
        }
        wait_rows(-1);
        __syncthreads();

        step(0, yes{}, yes{});
        int t = 1;
        for (; t < n_full; ++t) step(t, no{}, no{});
        for (; t < ntiles; ++t) step(t, yes{}, no{});
        int sc[2] = {0, 0};
        pv_prep(sc);
        pv_mma(tile_ptr(ntiles - 1), sc);
    }

    // ---- epilogue: lane (n32, h) of block j holds columns 32 (wave + 8 j) + 8 q + 4 h + i of
    // row 32 rb + n32, i = 0..3, for q = 0..3
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int rl = 32 * rb + n32;
        if (rl >= nrows) continue;
        const int64_t row = int64_t(b) * a.rows_per_req + row0 + rl;
        const float inv = lc[rb] > 0.f ? a.out_scale / lc[rb] : 0.f;
        const float lse2 = le[rb] > 0.f ? float(mc[rb]) + __log2f(le[rb]) : kNegInf;
#pragma unroll
        for (int j = 0; j < kMyBlocks; ++j) {
            if (j == 1 && !has_blk1) continue;
            const int cbase = 32 * (wave + 8 * j) + 4 * h;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float v0 = oacc[rb][j][4 * q] * inv, v1 = oacc[rb][j][4 * q + 1] * inv;
                const float v2 = oacc[rb][j][4 * q + 2] * inv, v3 = oacc[rb][j][4 * q + 3] * inv;
                if (DIRECT) {
                    *reinterpret_cast<uint2 *>(a.out + row * DV + cbase + 8 * q) =
                        make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                } else {
                    *reinterpret_cast<f32x4 *>(a.part_o + (row * a.np + part) * DV + cbase + 8 * q) =
                        f32x4{v0, v1, v2, v3};
                }
            }
        }
        if (wave == 0 && h == 0) {
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
