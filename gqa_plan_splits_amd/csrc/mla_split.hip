// mla_split.hip -- split kernel of absorbed MLA decode for gfx950.
//
// What it computes (moonmath-amd README, "MLA decode"; Modular MAX planner page, MLA-style
// bullet): every key row of the pool is one fused row that serves as K (all DQK elements) and as
// V (its first DV elements), dequantized with one per-tensor kv_scale; rows are fp8 e4m3, or bf16
// (the bf16 cache the AITER issue "[Perf] pa_decode_sparse" offers to re-measure on, in its
// closing paragraph).  A CTA owns up to 64
// query rows of one request and walks one partition of that request's keys, writing the
// partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.  Under
// decode context parallelism (same README section) the call holds one rank's share of each
// request's positions, and the draft window is taken on the global positions.  A negative slot
// id is a skipped key (the top-k lists' has_invalid case, AITER issue "[Perf]
// pa_decode_sparse", Measurements): its position counts, its weight is zero.  With a second
// cache (FlashInfer sparse planner page, Parameters: extra_topk) a request's key list continues
// past its pool keys with its second-cache rows, of the same format and scale.
//
// Arithmetic.  QK^T multiplies the bf16 query by the stored fp8 K decoded exactly to bf16, on
// the bf16 MFMA: every product is exact and the sums are fp32.  (gfx950's block-scaled fp8 MFMA
// would run an exact fp8 hi/lo split of the query at the same speed, but it aligns its 128
// products to about 15 bits below the largest one, an error of order 2^-15 max|q k| on every
// score, which the base-2 LSE of a row with few keys or a peaky softmax shows directly.)  The
// softmax weights p = 2^(score - m + 8), m an integer reference at most kLazyMax below the
// ceiling of the row's largest base-2 score so far (it moves only when a block's maximum exceeds
// it by more than that), are stored as fp16 (11 significant bits); PV multiplies them by V
// decoded exactly to fp16 on the fp16 MFMA.  The output is normalized by the sum of the stored weights, so a dominant key
// carries no rounding of its own weight into it; the LSE comes from the sum of the exact ones.
// bf16 rows go to the bf16 MFMA as stored, and their value part is converted to fp16 (exact for
// magnitudes in fp16's normal range; the library requires stored values below 65520).
//
// Work split (512 threads = 8 waves, one CTA per CU; waves w and w + 4 share SIMD w & 3, so
// every SIMD runs one score wave and one value wave):
//   - Score waves 0, 2 (query rows 0-31) and 1, 3 (rows 32-63) hold their rows' queries in
//     registers and compute S^T = K Q^T on v_mfma_f32_32x32x16_bf16 for 32 keys at a time; the
//     two waves of the same rows take alternate 32-key blocks (fp8: the two halves of each 64-key
//     tile; bf16: alternate 32-key tiles) and each keeps its own online softmax of those blocks.
//     They hand the value waves each block's weights P (fp16) and integer maximum through LDS,
//     and their final sums at the end.
//   - Value waves 4-7 accumulate output columns 128 v .. 128 v + 127
//     (v = 0..3) of all 64 rows on v_mfma_f32_32x32x16_f16: V^T comes from the tile in LDS through
//     transposed reads (ds_read_b64_tr_b8 for fp8, ds_read_b64_tr_b16 for bf16) and is converted
//     to fp16, P^T from LDS; when a block's maximum is above the accumulators', they are first
//     scaled by the exact power of two 2^(m_old - m_new).  The value waves also move the data:
//     wave v copies its columns of every key of a tile (and a quarter of the rope tails of
//     576-wide rows) straight from HBM into LDS with global_load_lds_dwordx4, three tiles ahead,
//     after loading the tile's slot ids the same way three tiles before that.  The copies are
//     issued from inline assembly and waited for with explicit vmcnt counts (the compiler would
//     drain every copy in flight before each LDS read).
//   - One barrier per tile.  The score waves run one tile ahead of the value waves: in step t
//     they compute the softmax of tile t and the scores of tile t + 1 (fp8: each wave both,
//     interleaved; bf16: the owner of tile t its softmax while the other wave of its rows runs
//     the MFMAs of tile t + 1), while the value waves apply tile t - 1.  The value waves run at a
//     raised issue priority (s_setprio 1): their copies and PV MFMAs go out as soon as they are
//     ready, and the score wave of the SIMD, whose softmax and K conversions are most of the
//     CTA's vector work, fills the remaining issue slots.
//
// LDS (160 KiB): a four-slot ring of the key rows' first 512 elements and a three-slot ring of the
// 64-element rope tails of 576-wide rows (fp8 layout below; bf16 rows at swz16).  Line j (bytes 128 j .. 128 j + 127 of the rows) of a
// slot's 64 keys fills 8 KiB at j * 8192, tile position P at P * 128, its 16-byte chunks permuted
// by an XOR with swz_line(P) (bits 2, 1 and 3 of P); a tail slot holds position P at P * 64,
// chunks permuted with bit 2 of P.  A copy instruction writes 1 KiB of consecutive 16-byte slots,
// so it moves whole 128-byte lines: one line of 8 keys (positions 8 i .. 8 i + 7 hold keys i,
// 8 + i, .., 56 + i of the tile, so that each lane's keys over the 8 instructions are consecutive
// in the slot list), or 16 rope tails.
//
// Bank conflicts.  gfx950's LDS has 64 four-byte banks.  Measured with the SQ_LDS_BANK_CONFLICT
// counter on probe patterns: a ds_read_b128 is served in four cycles of 16 lanes, lane l in cycle
// (l >> 5, parity of bits 2..4 of l); a ds_read_b64 (also the transposing ds_read_b64_tr_b8) in
// two cycles of 32 lanes, l < 32 and l >= 32.  A cycle is conflict-free when its lanes touch
// distinct 16-byte (8-byte) slots of a 256-byte bank row, or share an address.  The permutations
// above satisfy that for the score-operand reads (16 keys x one chunk pair per instruction), the
// transposed value reads (8 keys x chunks c and c ^ 4) and the rope-tail reads at once; the plain
// (P >> 1) & 7 permutation left the score reads two-way conflicted.
#include "device_common.hpp"
#include "kernels.hpp"
#include "mla_common.hpp"

#include <type_traits>

namespace gqa {
namespace {

// EXTRA: a second cache (the sparse planner page's extra_topk): request b's keys are its
// seq_lens[b] pool keys and then its second-cache rows; a key's list position picks the cache.
template <int DQK, int DV, bool DIRECT, bool EXTRA, bool KV16>
__global__ void __launch_bounds__(kThreads, 1) mla_split_kernel(const MlaSplitArgs a) {
    using T = MlaLayout<DQK, KV16>;
    constexpr int DLAT = DQK - 64;
    constexpr int kBK = T::kBK;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T::kLdsBytes];

    const int logical = xcd_logical_block(blockIdx.x, a.total_ctas);
    if (logical < 0) return;
    const int rblk = logical % a.row_blocks;
    const int rest = logical / a.row_blocks;
    // np equal partitions per request, or the planned length-proportional slots
    const int b = a.part_start ? request_of_slot(a.part_start, a.batch, rest) : rest / a.np;
    if (b >= a.batch) return;
    const int part = a.part_start ? rest - a.part_start[b] : rest % a.np;

    // Keys of this partition: ceil(S / np) rounded up to block_k, the last ones possibly empty;
    // no row of the block sees past the block's latest draft token.
    const int S1 = a.seq_lens[b];   // keys in the pool
    const int base = a.kv_indptr[b];
    const int base2 = EXTRA ? a.kv2_indptr[b] : 0;
    const int S = EXTRA ? S1 + (a.kv2_indptr[b + 1] - base2) : S1;
    // slot-id address of list position pos (< S) and whether the key is the second cache's
    auto id_ptr = [&](int pos) -> const int32_t * {
        return EXTRA && pos >= S1 ? a.kv2_indices + base2 + (pos - S1) : a.kv_indices + base + pos;
    };
    // Keys draft position t sees: 0 .. S - q_len + t, or under context parallelism the local keys
    // whose global positions j * cp_world + cp_rank are at most glen - q_len + t.
    const int G = a.cp_world > 1 ? a.glen[b] : S;
    auto visible = [&](int t) {
        const int last = G - a.q_len + t;   // last visible global position
        if (a.cp_world == 1) return max(0, last + 1);
        return last >= a.cp_rank ? min(S, (last - a.cp_rank) / a.cp_world + 1) : 0;
    };
    const int chunk = a.part_start ? a.part_chunk[b]
                                   : ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int row0 = rblk * kBM;
    const int nrows = min(kBM, a.rows_per_req - row0);
    const int k1 = min(visible((row0 + nrows - 1) / a.H), k0 + chunk);
    const int kfull = min(k1, visible(row0 / a.H));  // keys every row sees
    const int ntiles = k1 > k0 ? (k1 - k0 + kBK - 1) / kBK : 0;
    // Tiles whose keys every row of the block sees need no mask.
    const int n_full = min(ntiles, max(0, (kfull - k0) / kBK));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 31, h = lane >> 5;   // 32x32 operand / result coordinates
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    uint8_t *const P = lds + T::kPOff;
    uint8_t *const ML = lds + T::kMlOff;
    const int32_t *const id_ring = reinterpret_cast<const int32_t *>(lds + T::kIdOff);
    uint64_t *const bad_ring = reinterpret_cast<uint64_t *>(lds + T::kBadOff);

    // Roles by wave: waves w and w + 4 share a SIMD.  Score waves 0-3 (rows 32 (w & 1) ..
    // + 31, block (w >> 1) of every tile) and value waves 4-7 (columns of line w - 4): one of
    // each per SIMD, so that the score waves' vector work (K conversions, softmax) spreads over
    // all four SIMDs.
    if (wave < 4) {
        // ================================ score wave ================================
        // Score wave w: query rows 32 (w & 1) .. + 31 against 32-key block kb = w >> 1 of every
        // tile, S^T = K Q^T on v_mfma_f32_32x32x16_bf16.  The stored fp8 K bytes are converted
        // exactly to bf16 in registers, so every product q * k is exact and the sums are fp32.
        // Lane (n, h) reads the 64 bytes 64 h .. 64 h + 63 of each 128-byte line of key n of the
        // block: MFMA j (0..7) of line L takes its bytes 8 j .. 8 j + 7 as k slots 8 h .. 8 h + 7,
        // dims 128 L + 64 h + 8 j + 0..7 (the query operand takes the same dims).  The 64-byte
        // rope tail of 576-byte rows is four more MFMAs over dims 512 + 32 h + 8 j + 0..7.  The
        // two score waves of the same rows run alternate blocks, so each keeps its own
        // online softmax; the value waves align the two, and merge their sums at the end.
        // In the MFMA output layout lane (n, h) holds row n's scores of block positions
        // 8 j + 4 h + i (j, i = 0..3).  bf16 rows: block kb is every other 32-key tile (t = kb
        // mod 2), and lane (n, h) reads elements 32 h .. 32 h + 31 of each 64-element line, one
        // 16-byte chunk (8 dims) per MFMA, the rope tail as a ninth line.
        const int kb = wave >> 1;               // this wave's block of every tile
        const int srow = 32 * (wave & 1) + n;   // row within the CTA
        const bool row_ok = srow < nrows;
        constexpr int NL = DQK / 128;           // full 128-byte lines per fp8 row
        // MFMAs per 32-key block: fp8, 8 per 128-byte line and 4 for the rope tail; bf16, 4 per
        // 64 elements
        constexpr int NQ = KV16 ? 4 * (DQK / 64) : 8 * NL + (T::kTail ? 4 : 0);
        int p_end;                              // keys visible to this row
        const float c_row = a.score_scale;      // base-2 score per unit of the raw product
        bf16x8 qv[NQ];                          // B operands: this lane's query dims per MFMA
        {
            const int r = row0 + srow;
            const int t = row_ok ? r / a.H : 0;
            const int hh = row_ok ? r - t * a.H : 0;
            p_end = row_ok ? min(visible(t), k1) : k0;
            const int64_t tok = int64_t(b) * a.q_len + t;
            const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(hh) * a.q_st_head;
            const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(hh) * a.qpe_st_head;
            auto piece = [&](int d) {
                return as_bf16x8(row_ok ? load_q8<DLAT>(ql, qp, d) : u32x4{0u, 0u, 0u, 0u});
            };
            if constexpr (KV16) {
#pragma unroll
                for (int L = 0; L < DQK / 64; ++L)
#pragma unroll
                    for (int j = 0; j < 4; ++j) qv[4 * L + j] = piece(64 * L + 32 * h + 8 * j);
            } else {
#pragma unroll
                for (int L = 0; L < NL; ++L)
#pragma unroll
                    for (int j = 0; j < 8; ++j) qv[8 * L + j] = piece(128 * L + 64 * h + 8 * j);
                if constexpr (T::kTail) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) qv[8 * NL + j] = piece(512 + 32 * h + 8 * j);
                }
            }
        }

        // LDS offsets of this lane's K operand within tile t's slots: key at position 32 kb + n,
        // chunks 4 h .. 4 h + 3 of each line (line L adds 8192 bytes), rope-tail chunks 2 h and
        // 2 h + 1.
        // (bf16 rows: key at position n of the 32-key tile, chunks 4 h .. 4 h + 3 of each line
        // and of the rope tail, each chunk 8 dims of one MFMA.)
        int k_off[4], k_tail[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) k_off[c] = KV16 ? line_off16(0, n, 4 * h + c) : line_off(0, 32 * kb + n, 4 * h + c);
#pragma unroll
        for (int c = 0; c < 2; ++c) k_tail[c] = T::kTailOff + tail_off(32 * kb + n, 2 * h + c);
        // Slot-list index of this lane's score (j, i), relative to the tile: fp8,
        // key_of_pos(32 kb + 8 j + 4 h + i) = 32 h + 8 i + 4 kb + j; bf16,
        // key_of_pos16(8 j + 4 h + i) = 16 h + 4 i + j.
        const int kidx = KV16 ? 16 * h : 32 * h + 4 * kb;
        constexpr int kIStride = KV16 ? 4 : 8;

        // K operand reads (line L of tile t: 4 chunks; the rope tail: 2), and their exact
        // conversion to bf16 with the MFMAs of this wave's block, in one accumulator chain (the
        // matrix core forwards an accumulator to the next MFMA of the same kind): line L (8
        // MFMAs), and the rope tail (4 MFMAs).  The reads are issued a stage before their MFMAs.
        auto k_load = [&](int t, int L, u32x4 (&kr)[4]) {
            const uint8_t *lb = lds + (t % kLineSlots) * 32768 + 8192 * L;
#pragma unroll
            for (int c = 0; c < 4; ++c) kr[c] = *reinterpret_cast<const u32x4 *>(lb + k_off[c]);
        };
        auto qk_regs = [&](int L, const u32x4 (&kr)[4], f32x16 &acc) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[c].x, kr[c].y), qv[8 * L + 2 * c], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[c].z, kr[c].w), qv[8 * L + 2 * c + 1], acc, 0, 0, 0);
            }
        };
        auto tail_load = [&](int t, u32x4 (&kr)[2]) {
            const uint8_t *tlb = lds + (t % kTailSlots) * 4096;
#pragma unroll
            for (int c = 0; c < 2; ++c) kr[c] = *reinterpret_cast<const u32x4 *>(tlb + k_tail[c]);
        };
        auto tail_regs = [&](const u32x4 (&kr)[2], f32x16 &acc) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[c].x, kr[c].y), qv[8 * NL + 2 * c], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fp8x8_to_bf16x8(kr[c].z, kr[c].w), qv[8 * NL + 2 * c + 1], acc, 0, 0, 0);
            }
        };
        auto zero16 = [](f32x16 &x) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] = 0.f;
        };
        // bf16 rows: the scores of tile t, the stored K chunks straight into the bf16 MFMA, in two
        // accumulator chains (alternate 64-element lines) summed at the end.
        auto qk16 = [&](int t, f32x16 &acc) {
            f32x16 acc2;
            zero16(acc);
            zero16(acc2);
#pragma unroll
            for (int L = 0; L < DQK / 64; ++L) {
                const uint8_t *lb = L < 8 ? lds + (t % kLineSlots) * 32768 + 4096 * L
                                          : lds + T::kTailOff + (t % kTailSlots) * 4096;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const u32x4 k16 = *reinterpret_cast<const u32x4 *>(lb + k_off[c]);
                    if (L & 1)
                        acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k16), qv[4 * L + c], acc2, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(k16), qv[4 * L + c], acc, 0, 0, 0);
                }
            }
            acc += acc2;
        };

        // Online softmax over this wave's blocks, in base 2 with an integer reference maximum m (at
        // most kLazyMax below the ceiling of the largest base-2 score so far): a key's weight is
        // p = 2^(score - m + 8) in (0, 2^(8 + kLazyMax)], stored in fp16 (11 significant bits).  The row's sums of the stored weights
        // (lq, which normalizes the output: a dominant key then carries no rounding of its own
        // weight into it) and of the exact weights (le, which gives the log-sum-exp) are rescaled
        // by the exact power of two 2^(m_old - m_new) when m moves.  Lanes n and n + 32 hold the
        // same values.  The block's maximum goes to LDS beside P.  The work comes in four stages,
        // each placed beside the MFMAs of one 128-byte line of the next tile's scores.
        int m_run = kNoMax;
        float lq_run = 0.f, le_run = 0.f;
        struct Soft {
            float alpha, bias, esum, qsum;
            int m;
        };
        // stage 0: masks (the masked variant: tiles past some row's window or the partition end,
        // and tiles with skipped keys, whose scores of keys a row does not see become -inf), the
        // block maximum and the new running maximum
        auto sm0 = [&](int t, f32x16 &sc, auto masked) -> Soft {
            if constexpr (decltype(masked)::value) {
                // keys whose slot id is negative (bit k: slot-list index k of the tile)
                const uint32_t bad = uint32_t(bad_ring[t % kIdSlots] >> kidx);
                const int thr = p_end - k0 - t * kBK - kidx;   // visible: index < thr
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (((bad >> (kIStride * i + j)) & 1) || kIStride * i + j >= thr) sc[4 * j + i] = kNegInf;
            }
            float mx = sc[0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sc[i]);
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            const int mt = mx == kNegInf ? kNoMax : int(ceilf(mx * c_row));
            // The reference maximum m is at least the other score wave's of the same rows (as
            // published after its step t - 1), so that the two blocks of a tile mostly share it
            // and the value waves rarely align them; it moves to mt only when a block's maximum
            // exceeds it by more than kLazyMax, so that the accumulators are rarely rescaled.
            // The weights then lie in (0, 2^(8 + kLazyMax)], inside fp16's range.
            const int m_other = t > 0 ? *reinterpret_cast<const int *>(
                                            ML + ((t - 1) & 1) * T::kMlBytes + 256 * (1 - kb) + srow * 4)
                                      : kNoMax;
            Soft sf;
            sf.m = max(m_run, m_other);
            if (mt > sf.m + kLazyMax) sf.m = mt;
            sf.alpha = ldexpf(1.f, m_run - sf.m);
            sf.bias = float(8 - sf.m);
            sf.esum = sf.qsum = 0.f;
            return sf;
        };
        // stages 1 and 2: the weights of score groups j0, j0 + 1 (8 per lane) to P
        auto sm12 = [&](int t, int j0, const f32x16 &sc, Soft &sf) {
            uint8_t *pb = P + (t & 1) * 8192;
#pragma unroll
            for (int j = j0; j < j0 + 2; ++j) {
                const float p0 = fast_exp2(fmaf(sc[4 * j], c_row, sf.bias));
                const float p1 = fast_exp2(fmaf(sc[4 * j + 1], c_row, sf.bias));
                const float p2 = fast_exp2(fmaf(sc[4 * j + 2], c_row, sf.bias));
                const float p3 = fast_exp2(fmaf(sc[4 * j + 3], c_row, sf.bias));
                const f16x2 h01 = pack_f16x2(p0, p1), h23 = pack_f16x2(p2, p3);
                sf.esum += (p0 + p1) + (p2 + p3);
                // the stored weights' sum: v_dot2_f32_f16 against (1, 1) adds two fp16 values
                // to an fp32 sum (exact products)
                sf.qsum = __builtin_amdgcn_fdot2(h01, f16x2{1.0f16, 1.0f16}, sf.qsum, false);
                sf.qsum = __builtin_amdgcn_fdot2(h23, f16x2{1.0f16, 1.0f16}, sf.qsum, false);
                *reinterpret_cast<u32x2 *>(pb + p_slot(srow, (KV16 ? 0 : 4 * kb) + j) + 8 * h) =
                    u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
            }
        };
        // stage 3: the row sums, the running state, the block maximum to LDS
        auto sm3 = [&](int t, Soft &sf) {
            const auto se = __builtin_amdgcn_permlane32_swap(__float_as_uint(sf.esum), __float_as_uint(sf.esum), false, false);
            const auto sq = __builtin_amdgcn_permlane32_swap(__float_as_uint(sf.qsum), __float_as_uint(sf.qsum), false, false);
            lq_run = fmaf(lq_run, sf.alpha, __uint_as_float(sq[0]) + __uint_as_float(sq[1]));
            le_run = fmaf(le_run, sf.alpha, __uint_as_float(se[0]) + __uint_as_float(se[1]));
            m_run = sf.m;
            // lanes n and n + 32 hold the same value and both store it (no branch)
            *reinterpret_cast<int *>(ML + (t & 1) * T::kMlBytes + 256 * kb + srow * 4) = m_run;
        };
#define GQA_SB __builtin_amdgcn_sched_barrier(0)

        // Step t: the softmax of tile t (whose scores `cur` holds) in four stages, each beside the
        // MFMAs of one line of tile t + 1's scores (the last tile again at the end; those scores
        // are then unused), which accumulate in `nxt`.  Each line's K bytes are read during the
        // stage before (line 0 and the rope tail before the first stage's softmax work), so the
        // LDS latency is not waited out in front of the MFMAs.
        auto step = [&](int t, f32x16 &cur, f32x16 &nxt, auto masked) {
            const int tq = min(t + 1, ntiles - 1);
            u32x4 ka[4], kb2[4], kt[2];
            zero16(nxt);
            k_load(tq, 0, ka);
            if constexpr (T::kTail) tail_load(tq, kt);
            Soft sf = sm0(t, cur, masked);
            k_load(tq, 1, kb2);
            if constexpr (T::kTail) tail_regs(kt, nxt);
            qk_regs(0, ka, nxt);
            GQA_SB;
            sm12(t, 0, cur, sf);
            k_load(tq, 2, ka);
            qk_regs(1, kb2, nxt);
            GQA_SB;
            sm12(t, 2, cur, sf);
            k_load(tq, 3, kb2);
            qk_regs(2, ka, nxt);
            GQA_SB;
            sm3(t, sf);
            qk_regs(3, kb2, nxt);
            __syncthreads();   // P(t) published; tile t + 2 landed
        };

        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        // tiles with keys past some row's window or the partition end, or with skipped keys (mask
        // published when the tile's copies were issued), take the masked variant
        auto masked_tile = [&](int t) {
            return t >= n_full || __builtin_amdgcn_readfirstlane(uint32_t(bad_ring[t % kIdSlots] != 0));
        };
        if constexpr (KV16) {
            // bf16 rows: the two score waves of the same rows take alternate tiles (wave kb the tiles
            // t = kb mod 2) and alternate between two kinds of step: in step t the owner of tile t
            // runs its softmax (P(t) and the block maximum to LDS) while the other wave computes
            // the scores of tile t + 1 on the matrix core.
            if (ntiles > 0) {
                __syncthreads();   // tile 0 landed
                f32x16 sc;
                if (kb == 0) qk16(0, sc);
                __syncthreads();   // tile 1 landed; tile 0's rope tails read (step 0 refills their slot)
                for (int t = 0; t < ntiles; ++t) {
                    if ((t & 1) == kb) {
                        Soft sf = masked_tile(t) ? sm0(t, sc, yes{}) : sm0(t, sc, no{});
                        sm12(t, 0, sc, sf);
                        sm12(t, 2, sc, sf);
                        sm3(t, sf);
                    } else if (t + 1 < ntiles) {
                        qk16(t + 1, sc);
                    }
                    __syncthreads();   // P(t) published; tile t + 2 landed
                }
                uint8_t *fin = P + (ntiles & 1) * 8192 + kb * 768 + srow * 4;
                *reinterpret_cast<int *>(fin) = m_run;
                *reinterpret_cast<float *>(fin + 256) = lq_run;
                *reinterpret_cast<float *>(fin + 512) = le_run;
                __syncthreads();   // final states published
            }
            return;
        }
        if (ntiles > 0) {
            __syncthreads();   // tile 0 landed
            f32x16 sa, sb;
            zero16(sa);
            if constexpr (T::kTail) {
                u32x4 kt[2];
                tail_load(0, kt);
                tail_regs(kt, sa);
            }
#pragma unroll
            for (int L = 0; L < NL; ++L) {
                u32x4 kr[4];
                k_load(0, L, kr);
                qk_regs(L, kr, sa);
            }
            __syncthreads();   // tile 1 landed; tile 0's rope tails read (step 0 refills their slot)
            int t = 0;
            for (; t + 1 < ntiles; t += 2) {
                if (masked_tile(t)) step(t, sa, sb, yes{}); else step(t, sa, sb, no{});
                if (masked_tile(t + 1)) step(t + 1, sb, sa, yes{}); else step(t + 1, sb, sa, no{});
            }
            if (t < ntiles) {
                if (masked_tile(t)) step(t, sa, sb, yes{}); else step(t, sa, sb, no{});
            }
            // this wave's final state, in the P buffer the value waves no longer read:
            // [block][row] of {m, lq, le}
            uint8_t *fin = P + (ntiles & 1) * 8192 + kb * 768 + srow * 4;
            *reinterpret_cast<int *>(fin) = m_run;
            *reinterpret_cast<float *>(fin + 256) = lq_run;
            *reinterpret_cast<float *>(fin + 512) = le_run;
            __syncthreads();   // final states published
        }
#undef GQA_SB
        return;
    }

    // ================================ value wave ================================
    const int v = wave - 4;   // line v
    // raised issue priority on the SIMD it shares with a score wave
    __builtin_amdgcn_s_setprio(1);
    // ---- copies.  Instruction i writes tile positions 8 i .. 8 i + 7 of line v: lane L carries
    // slot-list key 8 (L >> 3) + i at position 8 i + (L >> 3), chunk position L & 7, i.e. global
    // chunk (L & 7) ^ swz_line(position).  The tail copy writes positions 16 v .. 16 v + 15.
    // Value wave 0 also loads every tile's slot ids into the shared id ring.
    // (bf16 rows: instruction i writes positions 8 (i & 3) .. + 7 of line 2 v + (i >> 2), lane L
    // key 4 (L >> 3) + (i & 3); the tail copy positions 8 v .. 8 v + 7.)
    const int jgrp = lane >> 3;
    const int tail_pos = KV16 ? 8 * v + jgrp : 16 * v + (lane >> 2);
    const int tail_chunk = KV16 ? 1024 + 16 * ((lane & 7) ^ swz16(tail_pos))
                                : 512 + 16 * ((lane & 3) ^ swz_tail(tail_pos));
    const int tail_key = KV16 ? key_of_pos16(tail_pos) : key_of_pos(tail_pos);
    // (row strides are below 2^32 bytes: one 32 x 32-bit product per row address)
    const uint32_t kv_stride = uint32_t(a.kv_stride);
    const bool id_loader = v == 0;

    auto issue_ids = [&](int tile) {
        if (id_loader && tile < ntiles)
            copy4(id_ptr(min(k0 + tile * kBK + lane, k1 - 1)),
                  lds_addr + T::kIdOff + (tile % kIdSlots) * 256);
    };
    // A negative slot id marks a key to skip: its copies read row 0 instead, and value wave 0
    // publishes the tile's mask of such keys for the score waves.
    // The copies of one tile given its slot ids: this lane's eight line keys 8 jgrp + i, its rope
    // tail key, and (value wave 0) the key numbered by the lane, whose sign makes the mask.
    // (a key's cache follows its list position, clamped like the id loads; both caches share the
    // row stride, so the second cache is the pool's address plus one offset)
    const int64_t kv2_delta = EXTRA ? int64_t(a.kv2 - a.kv) : 0;
    auto row_of = [&](int tile, int idx, int32_t id) -> const uint8_t * {
        const uint8_t *p = a.kv + uint64_t(uint32_t(max(id, 0))) * kv_stride;
        if (EXTRA && min(k0 + tile * kBK + idx, k1 - 1) >= S1) p += kv2_delta;
        return p;
    };
    // (kid: the ids of the lane's line keys 8 jgrp + i; bf16 rows, 4 jgrp + i for i < 4.  mid:
    // the id of the key numbered by the lane, or 0 past the tile's keys.)
    auto copy_lines = [&](int tile, const int32_t (&kid)[8], int32_t mid) {
        if (id_loader) {
            // every lane stores the same mask (no branch)
            const uint64_t bad = __builtin_amdgcn_ballot_w64(mid < 0);
            bad_ring[tile % kIdSlots] = bad;
        }
        if constexpr (KV16) {
            const uint32_t lslot = lds_addr + (tile % kLineSlots) * 32768 + v * 8192;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int line = 2 * v + (i >> 2), gi = i & 3;
                const int gc = (lane & 7) ^ swz16(8 * gi + jgrp);
                copy16(row_of(tile, 4 * jgrp + gi, kid[gi]) + 128 * line + 16 * gc,
                       lslot + 4096 * (i >> 2) + 1024 * gi);
            }
        } else {
            const uint32_t lslot = lds_addr + (tile % kLineSlots) * 32768 + v * 8192;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int gc = (lane & 7) ^ swz_line(8 * i + jgrp);
                copy16(row_of(tile, 8 * jgrp + i, kid[i]) + 128 * v + 16 * gc, lslot + 1024 * i);
            }
        }
    };
    auto copy_tail = [&](int tile, int32_t tid) {
        if (T::kTail)
            copy16(row_of(tile, tail_key, tid) + tail_chunk,
                   lds_addr + T::kTailOff + (tile % kTailSlots) * 4096 + 1024 * v);
    };
    // ... with the ids taken from the shared ring
    auto issue_lines = [&](int tile) {
        if (tile >= ntiles) return;
        const int32_t *ids = id_ring + (tile % kIdSlots) * 64;
        if constexpr (KV16) {
            const i32x4 ia = *reinterpret_cast<const i32x4 *>(ids + 4 * jgrp);
            const int32_t kid[8] = {ia.x, ia.y, ia.z, ia.w, 0, 0, 0, 0};
            copy_lines(tile, kid, lane < kBK ? ids[lane] : 0);
        } else {
            const i32x4 ia = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp);
            const i32x4 ib = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp + 4);
            const int32_t kid[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
            copy_lines(tile, kid, ids[lane]);
        }
    };
    auto issue_tail = [&](int tile) {
        if (!T::kTail || tile >= ntiles) return;
        copy_tail(tile, id_ring[(tile % kIdSlots) * 64 + tail_key]);
    };
    // Slot ids of tiles 0-2, straight from global memory into registers (so the first copies do
    // not wait on a workgroup barrier, which the score waves reach only after preparing Q).
    int32_t pre_kid[3][8], pre_tid[3], pre_mid[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const int kb = k0 + j * kBK;
        const int last = max(k1 - 1, k0);   // clamped like the ring's loads (k1 > k0 when used)
#pragma unroll
        for (int i = 0; i < 8; ++i) pre_kid[j][i] = 0;
        pre_tid[j] = pre_mid[j] = 0;
        if (j < ntiles) {
            if constexpr (KV16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) pre_kid[j][i] = *id_ptr(min(kb + 4 * jgrp + i, last));
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) pre_kid[j][i] = *id_ptr(min(kb + 8 * jgrp + i, last));
            }
            pre_tid[j] = *id_ptr(min(kb + tail_key, last));
            if (!KV16 || lane < kBK) pre_mid[j] = *id_ptr(min(kb + lane, last));
        }
    }
    // Schedule (tile j is read by the score waves in step j - 1, and by the value waves in
    // step j + 1 (576-byte fp8 rows: their V^T bytes at the end of step j); operations for
    // tiles >= ntiles are skipped, ids only in value wave 0):
    //   prologue: ids(3), rows(0), rows(1), rows(2), ids(4), ids(5);
    //   step t:   rows(t + 3) (lines and rope tails; the line slot held tile t - 1, whose values
    //             this wave has just applied or, V^T read ahead, holds in registers; the tail
    //             slot tile t), ids(t + 6), after the PV of tile t - 1 (before it for draft
    //             windows of 576-byte fp8 rows).
    // Copies retire in issue order.  Before the barrier that ends step t, tile t + 2 must have
    // landed (and with it ids(t + 4)); ids(t + 5) and step t's own issues may be outstanding.
    // The prologue's two barriers wait for tile 0 (whose scores the score waves compute between
    // them) and then tile 1.
    constexpr int NC = 8 + (T::kTail ? 1 : 0);
    auto cnt_rows = [&](int j) { return j >= 0 && j < ntiles ? NC : 0; };
    auto cnt_ids = [&](int j) { return id_loader && j >= 0 && j < ntiles ? 1 : 0; };
    auto issue_rows = [&](int tile) {
        issue_lines(tile);
        issue_tail(tile);
    };

    // ---- PV on v_mfma_f32_32x32x16_f16 as O^T = V^T P^T, four MFMAs per 64 keys.  V^T (A
    // operand) of column block cb: transposed read r hands lane (m, h) 8 fp8 bytes, keys
    // 16 h + 8 (r & 1) + 32 (r >> 1) + 0..7 of column m (a 16-lane group reads 8 keys of 16
    // columns: lane s = 2 k + hh points at key k of the read, bytes 8 hh.. of the chunk: cb for
    // lanes 0-15 of each half-wave, cb ^ 4 for lanes 16-31); converted exactly to fp16, they are
    // the k slots 8 h .. 8 h + 7 of MFMA r.  P^T (B operand) of MFMA r for row 32 rb + n: the
    // same keys' fp16 weights, P slot 2 h + (r & 1) + 4 (r >> 1) of the row.
    const int kk = (lane & 15) >> 1, hh = lane & 1, half = (lane >> 4) & 1;
    int v_off[4][4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r)
            v_off[cb][r] = line_off(v, 16 * h + 8 * (r & 1) + 32 * (r >> 1) + kk, half ? (cb ^ 4) : cb) + 8 * hh;
    int p_rd[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) p_rd[rb][r] = p_slot(32 * rb + n, 2 * h + (r & 1) + 4 * (r >> 1));
    // bf16 rows, two MFMAs per 32 keys.  V^T of column block cb (columns 128 v + 32 cb + 0..31,
    // line 2 v + (cb >> 1)): transposed read u of MFMA r (ds_read_b64_tr_b16) hands lane (m, h)
    // the bf16 values of keys 16 r + 8 h + 4 u + 0..3 of column m (a 16-lane group reads 4 keys x
    // 16 columns: lane s points at key s >> 2, columns 4 (s & 3) .. + 3 of its group's 16); the
    // two reads, converted to fp16, are the k slots 8 h .. 8 h + 7 of MFMA r.  P^T of MFMA r for
    // row 32 rb + n: P slot 2 r + h of the row.
    const int s16 = lane & 15, g16 = (lane >> 4) & 1;
    int v_off16[4][2][2];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int u = 0; u < 2; ++u)
                v_off16[cb][r][u] = line_off16(2 * v + (cb >> 1), 16 * r + 8 * h + 4 * u + (s16 >> 2),
                                               4 * (cb & 1) + 2 * g16 + ((s16 & 3) >> 1)) + 8 * (s16 & 1);
    int p_rd16[2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int r = 0; r < 2; ++r) p_rd16[rb][r] = p_slot(32 * rb + n, 2 * r + h);

    // The accumulators of rows n and 32 + n hold sums relative to mc[rb], the largest block
    // maximum applied so far.  A block whose maximum is larger first rescales them by the exact
    // power of two 2^(mc - m); one whose maximum is smaller has its fp16 weights scaled by
    // 2^(m - mc) (exact, or below 2^-24 of the row's largest weights, where they no longer count).
    int mc[2] = {kNoMax, kNoMax};
    f32x16 oacc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[rb][cb][i] = 0.f;

    // PV of tile t: every LDS read first (V^T bytes of both blocks, the weights, the block maxima),
    // so that their latency overlaps; then, block by block, the alignment of maxima, the exact
    // fp8 -> fp16 conversion of V and 16 MFMAs.
    int2v raw[4][4];   // [cb][r]: MFMA r's V^T bytes of column block cb
    auto read_vt = [&](int t) {
        const uint8_t *lb = lds + (t % kLineSlots) * 32768;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                raw[cb][r] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(lb + v_off[cb][r]));
    };
    // 576-byte rows: the V^T bytes of tile t are read at the end of step t, after the copies are
    // issued, so their latency passes during the wait for the barrier instead of in front of
    // the PV MFMAs of step t + 1 (512-byte rows read them in pv: holding them across the
    // barrier there costs spills).
    constexpr bool kVtAhead = T::kTail;
    auto pv = [&](int t) {
        if constexpr (!kVtAhead) read_vt(t);
        const uint8_t *pbuf = P + (t & 1) * 8192;
        const uint8_t *mlb = ML + (t & 1) * T::kMlBytes;
        f16x8 pw[2][4];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                pw[rb][r] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(pbuf + p_rd[rb][r]));
        int mblk[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb)
                mblk[kb][rb] = *reinterpret_cast<const int *>(mlb + 256 * kb + (32 * rb + n) * 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const int m = mblk[kb][rb];
                if (m > mc[rb]) {
                    const float alpha = ldexpf(1.f, mc[rb] - m);
                    mc[rb] = m;
                    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                        for (int cb = 0; cb < 4; ++cb) oacc[rb][cb] *= alpha;
                    }
                }
                const _Float16 ps = static_cast<_Float16>(ldexpf(1.f, m - mc[rb]));
                if (__builtin_amdgcn_ballot_w64(ps != _Float16(1.f))) {
#pragma unroll
                    for (int r = 2 * kb; r < 2 * kb + 2; ++r) pw[rb][r] *= ps;
                }
            }
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                f16x8 vt[2];
#pragma unroll
                for (int r = 0; r < 2; ++r)
                    vt[r] = fp8x8_to_f16x8(uint32_t(raw[cb][2 * kb + r].x), uint32_t(raw[cb][2 * kb + r].y));
                // the two row blocks alternate, so no MFMA waits on the one just before it
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb)
                        oacc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[r], pw[rb][2 * kb + r], oacc[rb][cb], 0, 0, 0);
            }
        }
    };

    // PV of a bf16 tile t: its one block of weights (score wave t & 1), as in pv.
    auto pv16 = [&](int t) {
        const uint8_t *pbuf = P + (t & 1) * 8192;
        const uint8_t *mlb = ML + (t & 1) * T::kMlBytes + 256 * (t & 1);
        const uint8_t *lb = lds + (t % kLineSlots) * 32768;
        s16x4 raw[4][2][2];
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    raw[cb][r][u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(lb + v_off16[cb][r][u]));
        f16x8 pw[2][2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int r = 0; r < 2; ++r)
                pw[rb][r] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(pbuf + p_rd16[rb][r]));
        int mblk[2];
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) mblk[rb] = *reinterpret_cast<const int *>(mlb + (32 * rb + n) * 4);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int m = mblk[rb];
            if (m > mc[rb]) {
                const float alpha = ldexpf(1.f, mc[rb] - m);
                mc[rb] = m;
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) oacc[rb][cb] *= alpha;
                }
            }
            const _Float16 ps = static_cast<_Float16>(ldexpf(1.f, m - mc[rb]));
            if (__builtin_amdgcn_ballot_w64(ps != _Float16(1.f))) {
#pragma unroll
                for (int r = 0; r < 2; ++r) pw[rb][r] *= ps;
            }
        }
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
            f16x8 vt[2];
#pragma unroll
            for (int r = 0; r < 2; ++r) vt[r] = bf16x8_to_f16x8(raw[cb][r][0], raw[cb][r][1]);
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    oacc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt[r], pw[rb][r], oacc[rb][cb], 0, 0, 0);
        }
    };
    auto pv_tile = [&](int t) {
        if constexpr (KV16) pv16(t); else pv(t);
    };

    if (ntiles > 0) {
        wait_vmem(0);   // the slot ids of tiles 0-2 are in registers
        issue_ids(3);
#pragma unroll
        for (int j = 0; j < 3; ++j)
            if (j < ntiles) {
                copy_lines(j, pre_kid[j], pre_mid[j]);
                copy_tail(j, pre_tid[j]);
            }
        issue_ids(4);
        issue_ids(5);
        // ids(3) and rows(0) landed; issued after rows(0): rows(1), rows(2), ids(4), ids(5)
        wait_vmem(cnt_rows(1) + cnt_rows(2) + cnt_ids(4) + cnt_ids(5));
        __syncthreads();   // tile 0, the ids of tile 3 and the masks of tiles 0-2 landed
        wait_vmem(cnt_rows(2) + cnt_ids(4) + cnt_ids(5));
        __syncthreads();   // tile 1 landed; the score waves read tile 0 (its tail slot is refilled
                           // in step 0)
        // Draft windows (q_len > 1, whose row blocks of a partition read the same keys, mostly
        // from L2): with the V^T bytes read a step ahead, tile t - 1's slots are free when step t
        // starts, so its copies go out before the PV (measured faster there, slower at q_len 1).
        const bool copies_first = !KV16 && kVtAhead && a.q_len > 1;
        for (int t = 0; t < ntiles; ++t) {
            if (copies_first) {
                issue_rows(t + 3);
                issue_ids(t + 6);
            }
            if (t > 0) pv_tile(t - 1);
            // line slot (t + 3) % 4 held tile t - 1 and tail slot (t + 3) % 3 tile t: every read
            // of them is done (the score waves' before the previous barrier, this wave's own
            // line just above)
            if (!copies_first) {
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_rows(t + 3);
                issue_ids(t + 6);
            }
            // tile t's line slot is refilled only in step t + 1, after its PV
            if constexpr (!KV16 && kVtAhead) read_vt(t);
            // rows(t + 2) and ids(t + 4) landed: everything issued before ids(t + 5) (value wave
            // 0) or before rows(t + 3) (the others)
            wait_vmem(cnt_ids(t + 5) + cnt_rows(t + 3) + cnt_ids(t + 6));
            __syncthreads();   // P(t) published; tile t + 2 landed
        }
        pv_tile(ntiles - 1);
        __syncthreads();   // the score waves' final states published
    }

    // ---- epilogue: lane (n, h) of block cb holds columns m = 8 q + 4 h + 0..3 of row 32 rb + n;
    // fp8, m < 16 lie in chunk cb of line v, the others in chunk cb ^ 4; bf16, column 32 cb + m.
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int rl = 32 * rb + n;
        if (rl >= nrows) continue;
        const int64_t row = int64_t(b) * a.rows_per_req + row0 + rl;
        // partial row: [row, np] or, with planned slots, [slot, rows_per_req]
        const int64_t prow = a.part_start ? int64_t(rest) * a.rows_per_req + row0 + rl
                                          : row * a.np + part;
        // the row's sums: those of the two score waves (one per block of every tile), each
        // relative to its own maximum, brought to the accumulators' maximum mc
        float lq = 0.f, le = 0.f;
        if (ntiles > 0) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const uint8_t *fin = P + (ntiles & 1) * 8192 + kb * 768 + rl * 4;
                const float f = ldexpf(1.f, *reinterpret_cast<const int *>(fin) - mc[rb]);
                lq = fmaf(*reinterpret_cast<const float *>(fin + 256), f, lq);
                le = fmaf(*reinterpret_cast<const float *>(fin + 512), f, le);
            }
        }
        const float inv = lq > 0.f ? a.out_scale / lq : 0.f;
        const float lse2 = le > 0.f ? float(mc[rb] - 8) + __log2f(le) : kNegInf;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = KV16 ? 128 * v + 32 * cb + 8 * q + 4 * h
                                     : 128 * v + 16 * (q < 2 ? cb : (cb ^ 4)) + 8 * (q & 1) + 4 * h;
                if (col >= DV) continue;
                const float v0 = oacc[rb][cb][4 * q] * inv, v1 = oacc[rb][cb][4 * q + 1] * inv;
                const float v2 = oacc[rb][cb][4 * q + 2] * inv, v3 = oacc[rb][cb][4 * q + 3] * inv;
                if (DIRECT) {
                    *reinterpret_cast<uint2 *>(a.out + row * DV + col) =
                        make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                } else {
                    *reinterpret_cast<f32x4 *>(a.part_o + prow * DV + col) =
                        f32x4{v0, v1, v2, v3};
                }
            }
        if (v == 0 && h == 0) {
            if (DIRECT) {
                if (a.lse2_out) a.lse2_out[row] = lse2;
            } else {
                a.part_lse2[prow] = lse2;
            }
        }
    }
}

template <int DQK, int DV, bool EXTRA, bool KV16>
hipError_t launch_shape(const MlaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(kThreads);
    if (direct)
        hipLaunchKernelGGL((mla_split_kernel<DQK, DV, true, EXTRA, KV16>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mla_split_kernel<DQK, DV, false, EXTRA, KV16>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <bool KV16>
hipError_t launch_format(const MlaSplitArgs &a, int d_qk, int d_v, bool direct, hipStream_t s) {
    const bool extra = a.kv2 != nullptr;
    if (d_qk == 576 && d_v == 512)   // (the second cache is a sparse top-k feature: 512-wide rows)
        return extra ? hipErrorInvalidValue : launch_shape<576, 512, false, KV16>(a, direct, s);
    if (d_qk == 512 && d_v == 448)
        return extra ? launch_shape<512, 448, true, KV16>(a, direct, s)
                     : launch_shape<512, 448, false, KV16>(a, direct, s);
    return hipErrorInvalidValue;
}

}  // namespace

int mla_rows_per_cta() { return kBM; }

hipError_t launch_mla_split(const MlaSplitArgs &a, int d_qk, int d_v, bool kv_bf16, bool direct, hipStream_t s) {
    if (a.block_k != 32 && a.block_k != 64) return hipErrorInvalidValue;
    // 512-byte fp8 rows of one cache (the sparse top-k layout) run on mla_wide.hip's kernel, which
    // decodes each K byte once per CTA; it measured faster there, and slower on 576-byte rows
    if (!kv_bf16 && a.kv2 == nullptr && d_qk == 512 && a.cp_world == 1) return launch_mla_wide(a, d_qk, d_v, direct, s);
    return kv_bf16 ? launch_format<true>(a, d_qk, d_v, direct, s) : launch_format<false>(a, d_qk, d_v, direct, s);
}

}  // namespace gqa
