// mla_wide.hip -- split kernel of absorbed MLA decode for gfx950 over 512-byte fp8 rows of one
// cache (the sparse top-k layout: 448 latent and 64 rope elements per row), with score waves that
// each cover all 64 query rows, so that every K byte is decoded once per CTA.
//
// It computes what mla_split.hip computes for those rows (moonmath-amd README, "MLA decode";
// AITER issue "[Perf] pa_decode_sparse": head_dim 512 = 448 + 64, packed fp8 cache): a CTA owns
// up to 64 query rows of one request (or top-k query) and one partition of its keys and writes
// the partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores, with
// the same exact arithmetic (stored fp8 K decoded exactly to bf16 against the bf16 query, fp32
// sums; weights p = 2^(score - m + 8) stored as fp16 against V decoded exactly to fp16; the
// output normalized by the sum of the stored weights, the LSE from the sum of the exact ones; m
// an integer reference maximum, at most kLazyMax below the ceiling of the row's largest base-2
// score so far), the same draft window and skipped keys.  (Decode context
// parallelism is defined for 576-byte rows only; those never reach this kernel.)
//
// Why.  mla_split.hip holds a row's query in one score wave's registers, 32 rows per wave, so
// each K byte is decoded twice per CTA (once per 32-row half).  Here each score wave holds the
// query of all 64 rows (dims 0-255 in 128 registers, dims 256-511 in LDS in MFMA operand order)
// and scores a quarter of each tile's keys, so each K byte is decoded once.  That costs a slot of
// the tile ring (three here, four there), which loses on long requests; on the top-k shapes,
// whose CTAs walk 4 to 32 tiles, it measured faster.
//
// Work split (512 threads = 8 waves, one CTA per CU; waves w and w + 4 share SIMD w & 3):
//   - score wave q = 0..3 (waves 0-3): for each 64-key tile t, the scores of tile positions
//     16 q .. 16 q + 15 for all 64 rows, S^T = K Q^T on v_mfma_f32_16x16x32_bf16 (one
//     accumulator per 16-row block, each K operand decoded once and used by the four blocks);
//     each row's maximum over those keys to LDS; after the first barrier of the step, the tile's
//     maximum of each row from the four score waves, the running maximum, this wave's weights of
//     its 16 keys to the shared P tile (fp16) and its partial sums.  Every score wave computes
//     the same running maximum of a row, so the four share one P tile, and score wave 0
//     publishes the row maxima beside it.
//   - value wave v = 0..3 (waves 4-7): in step t the PV of tile t - 1 for output columns
//     128 v .. 128 v + 127 of all 64 rows on v_mfma_f32_32x32x16_f16 (V^T through
//     ds_read_b64_tr_b8 decoded to fp16, P^T from LDS), after scaling its accumulators by
//     2^(m_old - m_new) where a row's maximum grew; after the first barrier, the copies of tile
//     t + 2 (line v of every key, straight from HBM into LDS with global_load_lds_dwordx4,
//     non-temporal; value wave 0 also loads the slot ids three tiles ahead of those).
// Two barriers per step: the first publishes the score waves' maxima (and ends the value waves'
// reads of tile t - 1, whose ring slot then takes tile t + 2); the second publishes P(t) and
// tile t + 1.  On each SIMD the score wave's QK^T MFMAs of tile t and the value wave's PV MFMAs
// of tile t - 1 share the matrix core.
//
// Score operand positions: row i of score wave q's A operand is tile position
// 16 q + 4 ((4 - (i >> 2)) & 3) + (i & 3), and k group g reads chunk g (dims 0-63 of a 128-byte
// line) or 4 + g (dims 64-127); with the line ring layout of mla_split.hip this makes the score
// reads and the P writes free of bank conflicts (checked exhaustively against the measured bank
// model).  The backend keeps the MFMA accumulators in VGPRs here, so the score role (query
// registers) and the value role (output accumulators) share one budget of 256 registers per wave
// (two waves per SIMD).
#include "device_common.hpp"
#include "kernels.hpp"
#include "mla_common.hpp"

#include <type_traits>

namespace gqa {
namespace {

constexpr int kWSlots = 3;        // line ring: tiles t - 1 (PV), t (scores), t + 1
constexpr int kWideDqk = 512, kWideDv = 448;

struct WideLayout {
    // query dims 256..511 in MFMA operand order: block (rb, L - 2, m) holds 64 lanes x 16 bytes,
    // lane l's B operand at 16 l
    static constexpr int kQlOff = kWSlots * 32768;
    static constexpr int kPOff = kQlOff + 4 * 2 * 4 * 1024;                     // P [64][64] fp16
    static constexpr int kMrOff = kPOff + 8192;                          // running max [2][64 rows]
    static constexpr int kMlOff = kMrOff + 512;                                  // m [4 waves][64 rows]
    static constexpr int kIdOff = kMlOff + 1024;
    static constexpr int kBadOff = kIdOff + kIdSlots * 256;
    static constexpr int kLdsBytes = kBadOff + kIdSlots * 8;
    // the score waves' final partial sums [4 waves][64 rows] of {lq, le} reuse the m and id regions
    static constexpr int kFinOff = kMlOff;
    static_assert(kIdOff + kIdSlots * 256 - kFinOff >= 2048, "final sums");
    static_assert(kLdsBytes <= 160 * 1024, "LDS");
};

template <bool DIRECT>
__global__ void __launch_bounds__(kThreads, 1) mla_wide_kernel(const MlaSplitArgs a) {
    using T = WideLayout;
    constexpr int DV = kWideDv;
    constexpr int DLAT = kWideDqk - 64;
    constexpr int kBK = 64;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[T::kLdsBytes];

    const int logical = xcd_logical_block(blockIdx.x, a.total_ctas);
    if (logical < 0) return;
    const int rblk = logical % a.row_blocks;
    const int rest = logical / a.row_blocks;
    const int b = a.part_start ? request_of_slot(a.part_start, a.batch, rest) : rest / a.np;
    if (b >= a.batch) return;
    const int part = a.part_start ? rest - a.part_start[b] : rest % a.np;

    const int S = a.seq_lens[b];
    const int base = a.kv_indptr[b];
    auto id_ptr = [&](int pos) -> const int32_t * { return a.kv_indices + base + pos; };
    // keys draft position t sees
    auto visible = [&](int t) { return max(0, S - a.q_len + t + 1); };
    const int chunk = a.part_start ? a.part_chunk[b]
                                   : ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int row0 = rblk * kBM;
    const int nrows = min(kBM, a.rows_per_req - row0);
    const int k1 = min(visible((row0 + nrows - 1) / a.H), k0 + chunk);
    const int kfull = min(k1, visible(row0 / a.H));
    const int ntiles = k1 > k0 ? (k1 - k0 + kBK - 1) / kBK : 0;
    const int n_full = min(ntiles, max(0, (kfull - k0) / kBK));

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    uint8_t *const P = lds + T::kPOff;
    int *const MR = reinterpret_cast<int *>(lds + T::kMrOff);
    int *const ML = reinterpret_cast<int *>(lds + T::kMlOff);
    const int32_t *const id_ring = reinterpret_cast<const int32_t *>(lds + T::kIdOff);
    uint64_t *const bad_ring = reinterpret_cast<uint64_t *>(lds + T::kBadOff);
    float *const fin = reinterpret_cast<float *>(lds + T::kFinOff);

    if (wave < 4) {
        // ================================ score wave ================================
        const int q = wave;
        const float c_row = a.score_scale;
        // lane (col, g) of 16x16 block rb holds query row 16 rb + col and, in the output, tile
        // positions pq + 0..3; as A operand it reads key position pa
        const int col = lane & 15, g = lane >> 4;
        const int pq = 16 * q + 4 * ((4 - g) & 3);
        const int pa = 16 * q + 4 * ((4 - (col >> 2)) & 3) + (lane & 3);
        const int kidx = key_of_pos(pq);   // slot-list index of position pq + e: kidx + 8 e

        // Query of row 16 rb + col, line L, dims 128 L + 16 (4 hh + g) + 8 j + 0..7 (m = 2 hh + j):
        // lines 0 and 1 in registers (qv[rb][L][m]), lines 2 and 3 in LDS, score wave q filling
        // row block q's operands.
        auto q_row = [&](int rb, const uint16_t *&ql, const uint16_t *&qp) {
            const int rl = 16 * rb + col;
            const bool ok = rl < nrows;
            const int r = row0 + rl;
            const int t = ok ? r / a.H : 0;
            const int hh = ok ? r - t * a.H : 0;
            const int64_t tok = int64_t(b) * a.q_len + t;
            ql = a.q + tok * a.q_st_tok + int64_t(hh) * a.q_st_head;
            qp = a.q_pe + tok * a.qpe_st_tok + int64_t(hh) * a.qpe_st_head;
            return ok;
        };
        {
            // this wave's row block's LDS operands first (their loads then do not add to the
            // registers' peak)
            const uint16_t *ql, *qp;
            const bool ok = q_row(q, ql, qp);
#pragma unroll
            for (int L = 2; L < 4; ++L)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int d = 128 * L + 16 * (4 * (m >> 1) + g) + 8 * (m & 1);
                    *reinterpret_cast<u32x4 *>(lds + T::kQlOff + ((q * 2 + L - 2) * 4 + m) * 1024 + 16 * lane) =
                        ok ? load_q8<DLAT>(ql, qp, d) : u32x4{0u, 0u, 0u, 0u};
                }
        }
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 qv[4][2][4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) {
            const uint16_t *ql, *qp;
            const bool ok = q_row(rb, ql, qp);
#pragma unroll
            for (int L = 0; L < 2; ++L)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int d = 128 * L + 16 * (4 * (m >> 1) + g) + 8 * (m & 1);
                    qv[rb][L][m] = as_bf16x8(ok ? load_q8<DLAT>(ql, qp, d) : u32x4{0u, 0u, 0u, 0u});
                }
        }

        // scores of tile t: S^T (16 keys x 16 rows) per row block, walked in half-lines (16 K
        // bytes for two k steps of a line); the next half-line's bytes are read while the current
        // one's MFMAs run, and the query operands held in LDS (lines 2 and 3: 32 MFMAs, operand i
        // at block i) through a ring of six registers, six MFMAs ahead, the first six read during
        // lines 0 and 1
        const int ko0 = line_off(0, pa, g), ko1 = line_off(0, pa, 4 + g);
        constexpr int NLQ = 32;   // MFMAs with an LDS query operand
        // LDS block of the i-th such operand: line 2 + i / 16, m = (i / 4) % 4, rb = i % 4
        auto lq_off = [&](int i) { return T::kQlOff + (((i & 3) * 2 + (i >> 4)) * 4 + ((i >> 2) & 3)) * 1024; };
        const uint8_t *const qlane = lds + 16 * lane;
        auto qk = [&](int t, f32x4 (&sacc)[4]) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
            const uint8_t *lb = lds + (t % kWSlots) * 32768;
            // half-line hl: line hl / 2, chunk g (hl even) or 4 + g, for MFMAs m = 2 (hl & 1) + j
            auto k_half = [&](int hl) {
                return *reinterpret_cast<const u32x4 *>(lb + 8192 * (hl >> 1) + ((hl & 1) ? ko1 : ko0));
            };
            u32x4 kc = k_half(0);
            u32x4 qr[6];
#pragma unroll
            for (int i = 0; i < 6; ++i) qr[i] = *reinterpret_cast<const u32x4 *>(qlane + lq_off(i));
#pragma unroll
            for (int hl = 0; hl < 8; ++hl) {
                const bf16x8 kk[2] = {fp8x8_to_bf16x8(kc.x, kc.y), fp8x8_to_bf16x8(kc.z, kc.w)};
                if (hl + 1 < 8) kc = k_half(hl + 1);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        if (hl < 4) {
                            sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[j], qv[rb][hl >> 1][2 * (hl & 1) + j], sacc[rb], 0, 0, 0);
                        } else {
                            const int i = 16 * ((hl >> 1) - 2) + 4 * (2 * (hl & 1) + j) + rb;
                            const bf16x8 qo = as_bf16x8(qr[i % 6]);
                            if (i + 6 < NLQ) qr[i % 6] = *reinterpret_cast<const u32x4 *>(qlane + lq_off(i + 6));
                            sacc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[j], qo, sacc[rb], 0, 0, 0);
                        }
                    }
            }
        };

        // online softmax state (rows 16 rb + col; equal in the four g lanes); the running maximum
        // of tile t lives in MR[t & 1]
        float lq_s[4], le_s[4];
#pragma unroll
        for (int rb = 0; rb < 4; ++rb) lq_s[rb] = le_s[rb] = 0.f;
        if (q == 0) MR[64 + lane] = kNoMax;   // the maximum "before tile 0"
        float sv[4][4];
        using yes = std::integral_constant<bool, true>;
        using no = std::integral_constant<bool, false>;
        // masks (tiles past some row's window or the partition end, and tiles with skipped keys),
        // then each row's maximum over this wave's keys to LDS
        auto local_max = [&](int t, const f32x4 (&sacc)[4], auto masked) {
            const uint64_t bad64 = decltype(masked)::value ? bad_ring[t % kIdSlots] : 0;
            // keys of the tile row 16 rb + col sees (slot-list index < thr[rb]); recomputed in
            // the masked tiles only
            int thr[4] = {kBK, kBK, kBK, kBK};
            if constexpr (decltype(masked)::value) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int rl = 16 * rb + col;
                    const int p_end = rl < nrows ? min(visible((row0 + rl) / a.H), k1) : k0;
                    thr[rb] = p_end - k0 - t * kBK;
                }
            }
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sv[rb][e] = sacc[rb][e];
                    if constexpr (decltype(masked)::value) {
                        if (((bad64 >> (kidx + 8 * e)) & 1) || kidx + 8 * e >= thr[rb]) sv[rb][e] = kNegInf;
                    }
                }
                const float mx = rows4_max(fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3])));
                const int mt = mx == kNegInf ? kNoMax : int(ceilf(mx * c_row));
                if (g == 0) ML[q * 64 + 16 * rb + col] = mt;
            }
        };
        // the tile's maximum of each row, the running maximum, this wave's weights to P
        auto weights = [&](int t) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int rl = 16 * rb + col;
                const int mt = max(max(ML[rl], ML[64 + rl]), max(ML[128 + rl], ML[192 + rl]));
                const int m_old = MR[64 * ((t + 1) & 1) + rl];
                // the reference maximum moves only when the tile's exceeds it by more than
                // kLazyMax (weights are then at most 2^(8 + kLazyMax)), so rescales are rare
                const int m_new = mt > m_old + kLazyMax ? mt : m_old;
                const float alpha = ldexpf(1.f, m_old - m_new);
                const float bias = float(8 - m_new);
                const float p0 = fast_exp2(fmaf(sv[rb][0], c_row, bias));
                const float p1 = fast_exp2(fmaf(sv[rb][1], c_row, bias));
                const float p2 = fast_exp2(fmaf(sv[rb][2], c_row, bias));
                const float p3 = fast_exp2(fmaf(sv[rb][3], c_row, bias));
                const f16x2 h01 = pack_f16x2(p0, p1), h23 = pack_f16x2(p2, p3);
                // the stored weights' sum: v_dot2_f32_f16 against (1, 1) (exact products)
                float qsum = __builtin_amdgcn_fdot2(h01, f16x2{1.0f16, 1.0f16}, 0.f, false);
                qsum = __builtin_amdgcn_fdot2(h23, f16x2{1.0f16, 1.0f16}, qsum, false);
                const float esum = (p0 + p1) + (p2 + p3);
                *reinterpret_cast<u32x2 *>(P + p_slot(rl, pq >> 3) + 8 * ((pq >> 2) & 1)) =
                    u32x2{__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23)};
                lq_s[rb] = fmaf(lq_s[rb], alpha, rows4_sum(qsum));
                le_s[rb] = fmaf(le_s[rb], alpha, rows4_sum(esum));
                if (q == 0 && g == 0) MR[64 * (t & 1) + rl] = m_new;
            }
        };
        auto masked_tile = [&](int t) {
            return t >= n_full || __builtin_amdgcn_readfirstlane(uint32_t(bad_ring[t % kIdSlots] != 0));
        };

        if (ntiles > 0) {
            __syncthreads();   // tile 0, the masks of tiles 0 and 1 and the LDS query published
            // The query registers are used from here on: without these (empty) uses the
            // compiler would wait for their loads inside the loop.
#pragma unroll
            for (int rb = 0; rb < 4; ++rb)
#pragma unroll
                for (int L = 0; L < 2; ++L)
#pragma unroll
                    for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(qv[rb][L][m]));
            for (int t = 0; t < ntiles; ++t) {
                f32x4 sacc[4];
                qk(t, sacc);
                if (masked_tile(t)) local_max(t, sacc, yes{}); else local_max(t, sacc, no{});
                __syncthreads();   // maxima of tile t published; tile t - 1's PV done
                weights(t);
                __syncthreads();   // P(t) published; tile t + 1 landed
            }
            // this wave's partial sums, in the m / id regions (unused from here on)
            if (g == 0) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    fin[q * 64 + 16 * rb + col] = lq_s[rb];
                    fin[256 + q * 64 + 16 * rb + col] = le_s[rb];
                }
            }
            __syncthreads();   // final sums published
        }
        return;
    }

    // ================================ value wave ================================
    const int v = wave - 4;
    // ---- copies (as the value waves of mla_split.hip: value wave v copies line v)
    const int jgrp = lane >> 3;
    // (row strides are below 2^32 bytes: one 32 x 32-bit product per row address)
    const uint32_t kv_stride = uint32_t(a.kv_stride);
    const bool id_loader = v == 0;
    auto issue_ids = [&](int tile) {
        if (id_loader && tile < ntiles)
            copy4(id_ptr(min(k0 + tile * kBK + lane, k1 - 1)), lds_addr + T::kIdOff + (tile % kIdSlots) * 256);
    };
    // a negative slot id is a skipped key: its copies read row 0, and value wave 0 publishes the
    // tile's mask of such keys
    auto row_of = [&](int32_t id) -> const uint8_t * { return a.kv + uint64_t(uint32_t(max(id, 0))) * kv_stride; };
    auto copy_lines = [&](int tile, const int32_t (&kid)[8], int32_t mid) {
        if (id_loader) bad_ring[tile % kIdSlots] = __builtin_amdgcn_ballot_w64(mid < 0);
        const uint32_t lslot = lds_addr + (tile % kWSlots) * 32768 + v * 8192;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int gc = (lane & 7) ^ swz_line(8 * i + jgrp);
            copy16(row_of(kid[i]) + 128 * v + 16 * gc, lslot + 1024 * i);
        }
    };
    auto issue_rows = [&](int tile) {
        if (tile >= ntiles) return;
        const int32_t *ids = id_ring + (tile % kIdSlots) * 64;
        const i32x4 ia = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp);
        const i32x4 ib = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp + 4);
        const int32_t kid[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        copy_lines(tile, kid, ids[lane]);
    };
    constexpr int NC = 8;   // copy instructions per tile
    auto cnt_rows = [&](int j) { return j >= 0 && j < ntiles ? NC : 0; };
    auto cnt_ids = [&](int j) { return id_loader && j >= 0 && j < ntiles ? 1 : 0; };

    // slot ids of tiles 0 and 1 straight into registers
    int32_t pre_kid[2][8], pre_mid[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int kb = k0 + j * kBK;
        const int last = max(k1 - 1, k0);
#pragma unroll
        for (int i = 0; i < 8; ++i) pre_kid[j][i] = 0;
        pre_mid[j] = 0;
        if (j < ntiles) {
#pragma unroll
            for (int i = 0; i < 8; ++i) pre_kid[j][i] = *id_ptr(min(kb + 8 * jgrp + i, last));
            pre_mid[j] = *id_ptr(min(kb + lane, last));
        }
    }

    // ---- PV: lane (n, h) of 32x32 block (rb, cb) holds row 32 rb + n, columns of line v (as the
    // value waves of mla_split.hip).  Column block cb's V^T offsets are block 0's with 16 cb
    // XORed in (the chunk field); row block 1's P offsets are row block 0's plus 4096.
    const int n = lane & 31, h = lane >> 5;
    const int kk8 = (lane & 15) >> 1, hb = lane & 1, half = (lane >> 4) & 1;
    int v_off[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) v_off[r] = line_off(v, 16 * h + 8 * (r & 1) + 32 * (r >> 1) + kk8, half ? 4 : 0) + 8 * hb;
    const int p_rd = p_slot(n, 2 * h);   // key step r: XOR ((r & 1) + 4 (r >> 1)) << 4
    int mc[2] = {kNoMax, kNoMax};
    f32x16 oacc[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[rb][cb][i] = 0.f;

    // PV of tile t: the accumulators follow the running maximum published with P(t) (scaled by
    // the exact power of two 2^(m_old - m_new) where it grew), then 32 MFMAs
    auto pv = [&](int t) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int m = MR[64 * (t & 1) + 32 * rb + n];
            if (m > mc[rb]) {
                const float alpha = ldexpf(1.f, mc[rb] - m);
                mc[rb] = m;
                if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
                    for (int cb = 0; cb < 4; ++cb) oacc[rb][cb] *= alpha;
                }
            }
        }
        const uint8_t *lb = lds + (t % kWSlots) * 32768;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            int2v raw[4];
#pragma unroll
            for (int cb = 0; cb < 4; ++cb)
                raw[cb] = __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) int2v *)(lb + (v_off[r] ^ (16 * cb))));
            const int pr = p_rd ^ (((r & 1) + 4 * (r >> 1)) << 4);
            f16x8 pw[2];
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) pw[rb] = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(P + 4096 * rb + pr));
#pragma unroll
            for (int cb = 0; cb < 4; ++cb) {
                const f16x8 vt = fp8x8_to_f16x8(uint32_t(raw[cb].x), uint32_t(raw[cb].y));
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    oacc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vt, pw[rb], oacc[rb][cb], 0, 0, 0);
            }
        }
    };

    if (ntiles > 0) {
        // Issue order: ids(2), rows(0), ids(3), rows(1), ids(4); then in step t, after the first
        // barrier, rows(t + 2) (its line slot held tile t - 1) and ids(t + 5).  Before
        // the second barrier of step t, rows(t + 1) and ids(t + 3) must have landed: everything
        // issued before ids(t + 4).
        wait_vmem(0);   // slot ids of tiles 0 and 1 in registers
        issue_ids(2);
        copy_lines(0, pre_kid[0], pre_mid[0]);
        issue_ids(3);
        if (1 < ntiles) {
            copy_lines(1, pre_kid[1], pre_mid[1]);
        }
        issue_ids(4);
        // tile 0 and ids(2) landed: ids(3), rows(1), ids(4) may be outstanding
        wait_vmem(cnt_ids(3) + cnt_rows(1) + cnt_ids(4));
        __syncthreads();   // tile 0, ids(2), the masks of tiles 0 and 1 and the LDS query published
        for (int t = 0; t < ntiles; ++t) {
            if (t > 0) pv(t - 1);
            // every read of tile t - 1's line slot is done: this wave's just above, the score
            // waves' in step t - 1
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            __syncthreads();   // maxima of tile t published; tile t - 1's PV done
            issue_rows(t + 2);
            issue_ids(t + 5);
            wait_vmem(cnt_ids(t + 4) + cnt_rows(t + 2) + cnt_ids(t + 5));
            __syncthreads();   // P(t) published; tile t + 1 and ids(t + 3) landed
        }
        pv(ntiles - 1);
        __syncthreads();   // the score waves' final sums published
    }

    // ---- epilogue: lane (n, h) of block cb holds columns 8 qq + 4 h + 0..3 of the block's 32;
    // columns qq < 2 lie in chunk cb of line v, the others in chunk cb ^ 4
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int rl = 32 * rb + n;
        if (rl >= nrows) continue;
        const int64_t row = int64_t(b) * a.rows_per_req + row0 + rl;
        // partial row: [row, np] or, with planned slots, [slot, rows_per_req]
        const int64_t prow = a.part_start ? int64_t(rest) * a.rows_per_req + row0 + rl : row * a.np + part;
        // the row's sums: the four score waves' partial sums, all relative to the running maximum
        float lq = 0.f, le = 0.f;
        if (ntiles > 0) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                lq += fin[s * 64 + rl];
                le += fin[256 + s * 64 + rl];
            }
        }
        const float inv = lq > 0.f ? a.out_scale / lq : 0.f;
        const float lse2 = le > 0.f ? float(mc[rb] - 8) + __log2f(le) : kNegInf;
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int c = 128 * v + 16 * (qq < 2 ? cb : (cb ^ 4)) + 8 * (qq & 1) + 4 * h;
                if (c >= DV) continue;
                const float v0 = oacc[rb][cb][4 * qq] * inv, v1 = oacc[rb][cb][4 * qq + 1] * inv;
                const float v2 = oacc[rb][cb][4 * qq + 2] * inv, v3 = oacc[rb][cb][4 * qq + 3] * inv;
                if (DIRECT) {
                    *reinterpret_cast<uint2 *>(a.out + row * DV + c) = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
                } else {
                    *reinterpret_cast<f32x4 *>(a.part_o + prow * DV + c) = f32x4{v0, v1, v2, v3};
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

}  // namespace

hipError_t launch_mla_wide(const MlaSplitArgs &a, int d_qk, int d_v, bool direct, hipStream_t s) {
    if (a.block_k != 32 && a.block_k != 64) return hipErrorInvalidValue;
    if (a.kv2 != nullptr || d_qk != kWideDqk || d_v != kWideDv) return hipErrorInvalidValue;
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(kThreads);
    if (direct)
        hipLaunchKernelGGL((mla_wide_kernel<true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mla_wide_kernel<false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace gqa
