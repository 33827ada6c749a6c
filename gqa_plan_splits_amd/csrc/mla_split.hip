// mla_split.hip -- split kernel of absorbed MLA decode for gfx950.
//
// What it computes (moonmath-amd README, "MLA decode"; Modular MAX planner page, MLA-style
// bullet): every key row of the pool is one fused fp8 e4m3 row that serves as K (all DQK bytes)
// and as V (its first DV bytes), dequantized with one per-tensor kv_scale.  A CTA packs 32 query
// rows (BM = 32) of one request and walks one partition of that request's keys, writing the
// partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Layout of the work:
//   - 256 threads = 4 waves.  Waves 0/1 own query rows 0-15 / 16-31 of the CTA; waves 2/3 own
//     the same rows.  For QK^T each pair splits the DQK contraction in halves and adds the two
//     partial score tiles through LDS (both waves then hold identical scores); for PV each wave
//     of the pair owns half of the DV output columns.  Each wave thus holds half of Q and half of
//     the output accumulator, which keeps it near 160 VGPRs so two waves fit on every SIMD.
//   - Keys are processed in tiles of BK (32 or 64).  The CTA gathers a tile (16 bytes per lane,
//     consecutive lanes on consecutive chunks of a row, slot ids read a tile ahead) into
//     registers one tile ahead of the compute, then writes it to LDS row-major, once.
//   - QK^T (S^T = K Q^T) and PV (O^T = V^T P^T) run on v_mfma_f32_16x16x32_bf16.  K is read
//     16 bytes per lane; V is read from the same row-major tile with ds_read_b64_tr_b8, which
//     hands each lane 8 keys of one value column -- the K-major operand layout.  The fp8 bytes
//     are converted to bf16 exactly as they are read; kv_scale is folded into the score scale and
//     the output scale.
//   - Each lane owns one query row's column of the score tile, so the row max / sum take two
//     cross-lane exchanges and the online-softmax rescale is a per-lane multiply (skipped when no
//     row's maximum moved).
//
// LDS tile layout (chunk-major, swizzled): 16-byte chunk c of tile key k sits in slot
// c * BK + (k ^ 12 * bit4(k) ^ (c % 16)).  A score-operand read (16 consecutive keys, one chunk)
// is then one contiguous 256-byte block; a transposed value read (keys 4g..4g+3 and 16+4g..
// 16+4g+3 of a 32-key step) lands on 8 distinct 16-byte slots; and the gather's stores (one key,
// consecutive chunks) land on distinct banks.  All three are free of bank conflicts, and the
// tile needs no padding.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

typedef int int2v __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Byte offset of byte d of tile key `key` (see the layout note above).
template <int BK>
__device__ __forceinline__ int tile_pos(int key, int d) {
    const int c = d >> 4;
    return ((c * BK + (key ^ (((key >> 4) & 1) * 12) ^ (c & 15))) << 4) + (d & 15);
}

template <int BK, int DQK, int DV>
struct MlaTile {
    static constexpr int kThreads = 256;
    static constexpr int kDLat = DQK - 64;             // latent width; V = first DV columns
    static constexpr int kF8Chunks = 2;                // 128-wide fp8 QK chunks per wave
    static constexpr int kRopeSteps = (DQK - 512) / 32;  // bf16 k-steps past 512 bytes (wave 2/3)
    static constexpr int kHalfV = DV / 2;              // output columns per wave
    static constexpr int kVBlocks = kHalfV / 16;       // 16 or 14
    static constexpr int kSBlocks = BK / 16;           // 16-key score blocks per tile
    static constexpr int kPvSteps = BK / 32;           // 32-key PV steps per tile
    static constexpr int kChunks = DQK / 16;           // 16-byte chunks per key row
    static constexpr int kItems = BK * kChunks;        // chunks per tile
    static constexpr int kItemsPerThread = (kItems + kThreads - 1) / kThreads;
    static constexpr int kKBytes = BK * DQK;
    static constexpr int kSxBytes = 4 * kSBlocks * 64 * 16;   // partial score exchange
    static constexpr int kLdsBytes = kKBytes + kSxBytes;
    static_assert(DQK == 576 || DQK == 512, "row width");
    static_assert(DV % 32 == 0 && DV <= kDLat, "value width");
    static_assert(BK == 32 || BK == 64, "tile");
};

// Loads 8 bf16 query values at d (< DQK) of one row: the latent part from q, the rope part from
// q_pe.  8-element pieces never straddle the boundary (it is a multiple of 8).
template <int DLAT>
__device__ __forceinline__ u32x4 load_q8(const uint16_t *ql, const uint16_t *qp, int d) {
    return d < DLAT ? *reinterpret_cast<const u32x4 *>(ql + d)
                    : *reinterpret_cast<const u32x4 *>(qp + (d - DLAT));
}

template <int BK, int DQK, int DV, bool DIRECT>
__global__ void __launch_bounds__(256, 2) mla_split_kernel(const MlaSplitArgs a) {
    using T = MlaTile<BK, DQK, DV>;
    constexpr int IPT = T::kItemsPerThread;
    constexpr int NSB = T::kSBlocks;

    __shared__ __attribute__((aligned(16))) uint8_t lds[T::kLdsBytes];
    uint8_t *const kbuf = lds;
    f32x4 *const sx = reinterpret_cast<f32x4 *>(lds + T::kKBytes);

    const int logical = xcd_logical_block(blockIdx.x, a.total_ctas);
    if (logical < 0) return;
    const int rb = logical % a.row_blocks;
    const int rest = logical / a.row_blocks;
    const int part = rest % a.np;
    const int b = rest / a.np;

    // Keys of this partition: ceil(S / np) rounded up to the tile, the last ones possibly empty;
    // no row of the block sees past the block's widest draft window.
    const int S = a.seq_lens[b];
    const int base = a.kv_indptr[b];
    const int chunk = ((S + a.np - 1) / a.np + BK - 1) / BK * BK;
    const int k0 = part * chunk;
    const int row_lo = rb * 32;
    const int row_last = min(row_lo + 32, a.rows_per_req) - 1;
    const int block_keys = max(0, S - a.q_len + row_last / a.H + 1);
    const int k1 = min(block_keys, k0 + chunk);
    const int ntiles = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, grp = lane >> 4, col = lane & 15;
    const int rg = wave & 1, hf = wave >> 1;

    // The query row whose column this lane holds.
    const int r_in = row_lo + rg * 16 + col;
    const bool row_ok = r_in < a.rows_per_req;
    const int t = row_ok ? r_in / a.H : 0;
    const int h = row_ok ? r_in - t * a.H : 0;
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;
    const bool pair_active = row_lo + rg * 16 < a.rows_per_req;

    // Q^T for the fp8 score MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, unit scales): this wave's
    // two 128-wide chunks of the row (d = 256 hf .. 256 hf + 255).  Lane (col, grp) holds
    // d = 128 i + 32 grp .. +31 of chunk i.  A bf16 value has 8 significant bits, so with the row
    // scaled by a power of two into [128, 256) it is the sum of two e4m3 values (hi = nearest,
    // lo = the exact remainder) except for elements below 2^-12 of the row maximum, whose
    // remainders fall under e4m3's subnormal step.  K is used as stored (fp8), so no K value is
    // converted.  The 64-wide rope tail of 576-byte rows runs on bf16 MFMA in waves 2/3.
    const int dbase = hf * 256;
    i32x8 qhi[T::kF8Chunks], qlo[T::kF8Chunks];
    float qinv;
    bf16x8 qrope[T::kRopeSteps > 0 ? T::kRopeSteps : 1];
    {
        const int64_t tok = int64_t(b) * a.q_len + t;
        const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(h) * a.q_st_head;
        const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(h) * a.qpe_st_head;
        float qv[T::kF8Chunks][32];
        float mx = 0.f;
#pragma unroll
        for (int i = 0; i < T::kF8Chunks; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                u32x4 v = u32x4{0u, 0u, 0u, 0u};
                if (row_ok) v = load_q8<T::kDLat>(ql, qp, dbase + 128 * i + 32 * grp + 8 * e);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    qv[i][8 * e + 2 * w] = bf16_lo(v[w]);
                    qv[i][8 * e + 2 * w + 1] = bf16_hi(v[w]);
                    mx = fmaxf(mx, fmaxf(fabsf(qv[i][8 * e + 2 * w]), fabsf(qv[i][8 * e + 2 * w + 1])));
                }
            }
        mx = fmaxf(mx, xor_shuffle(mx, 16));
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        int ex = 0;
        if (mx > 0.f) frexpf(mx, &ex);             // mx = f * 2^ex, f in [0.5, 1)
        const float qs = ldexpf(1.f, 8 - ex);      // row maximum scaled into [128, 256)
        qinv = ldexpf(1.f, ex - 8);
#pragma unroll
        for (int i = 0; i < T::kF8Chunks; ++i)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const float x0 = qv[i][4 * w] * qs, x1 = qv[i][4 * w + 1] * qs;
                const float x2 = qv[i][4 * w + 2] * qs, x3 = qv[i][4 * w + 3] * qs;
                int hi = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
                hi = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, hi, true);
                typedef float f32x2 __attribute__((ext_vector_type(2)));
                const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
                const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
                int lo = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - h01.x, x1 - h01.y, 0, false);
                lo = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - h23.x, x3 - h23.y, lo, true);
                qhi[i][w] = hi;
                qlo[i][w] = lo;
            }
#pragma unroll
        for (int s = 0; s < T::kRopeSteps; ++s) {
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (row_ok && hf == 1) v = load_q8<T::kDLat>(ql, qp, 512 + 32 * s + 8 * grp);
            qrope[s] = as_bf16x8(v);
        }
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[T::kVBlocks];
#pragma unroll
    for (int v = 0; v < T::kVBlocks; ++v) oacc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Gather: item i = tid + 256 u is chunk (i % kChunks) of tile key (i / kChunks).  Keys past
    // the partition end are clamped to its last key: their rows are real (finite) data, their
    // scores are masked to -inf and their probabilities are 0, so nothing is predicated -- the
    // loads stay unconditional and the slot-id loads never stall the wave before the compute.
    u32x4 stg[IPT];
    int idx[IPT];
    int ichunk[IPT], ikey[IPT];   // loop-invariant: chunk and tile key of each gather item
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
        const int item = min(tid + u * T::kThreads, T::kItems - 1);
        ichunk[u] = 16 * (item % T::kChunks);
        ikey[u] = item / T::kChunks;
    }
    const bool last_item_ok = tid + (IPT - 1) * T::kThreads < T::kItems;

#define GQA_LOAD_INDICES(tile)                                                                \
    _Pragma("unroll") for (int u = 0; u < IPT; ++u)                                           \
        idx[u] = a.kv_indices[base + min(k0 + (tile) * BK + ikey[u], k1 - 1)];
#define GQA_LOAD_ROWS()                                                                       \
    _Pragma("unroll") for (int u = 0; u < IPT; ++u)                                           \
        stg[u] = *reinterpret_cast<const u32x4 *>(a.kv + int64_t(idx[u]) * a.kv_stride + ichunk[u]);

    if (ntiles > 0) {
        GQA_LOAD_INDICES(0)
        GQA_LOAD_ROWS()
        if (ntiles > 1) { GQA_LOAD_INDICES(1) }
    }

    for (int it = 0; it < ntiles; ++it) {
        __syncthreads();
#pragma unroll
        for (int u = 0; u < IPT; ++u)
            if (u + 1 < IPT || last_item_ok)
                *reinterpret_cast<u32x4 *>(kbuf + tile_pos<BK>(ikey[u], ichunk[u])) = stg[u];
        __syncthreads();
        if (it + 1 < ntiles) {
            GQA_LOAD_ROWS()
            if (it + 2 < ntiles) { GQA_LOAD_INDICES(it + 2) }
        }

        // Partial S^T over this wave's half of the row: block j covers keys 16j..16j+15; lane
        // holds keys 16j+4grp+i of row col.
        f32x4 sacc[NSB];
        if (pair_active) {
#pragma unroll
            for (int j = 0; j < NSB; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            // the operands of two score blocks are read first, so the LDS latency is paid once
            // per pair of blocks rather than once per MFMA
#pragma unroll
            for (int j0 = 0; j0 < NSB; j0 += 2) {
                i32x8 kraw[2][T::kF8Chunks];
#pragma unroll
                for (int jj = 0; jj < 2; ++jj)
#pragma unroll
                    for (int i = 0; i < T::kF8Chunks; ++i) {
                        const int key = 16 * (j0 + jj) + col;
                        const int d = dbase + 128 * i + 32 * grp;
                        const u32x4 lo16 = *reinterpret_cast<const u32x4 *>(kbuf + tile_pos<BK>(key, d));
                        const u32x4 hi16 = *reinterpret_cast<const u32x4 *>(kbuf + tile_pos<BK>(key, d + 16));
                        kraw[jj][i] = i32x8{int(lo16.x), int(lo16.y), int(lo16.z), int(lo16.w),
                                            int(hi16.x), int(hi16.y), int(hi16.z), int(hi16.w)};
                    }
#pragma unroll
                for (int i = 0; i < T::kF8Chunks; ++i) {
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
                        sacc[j0 + jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            kraw[jj][i], qhi[i], sacc[j0 + jj], 0, 0, 0, 127, 0, 127);
#pragma unroll
                    for (int jj = 0; jj < 2; ++jj)
                        sacc[j0 + jj] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            kraw[jj][i], qlo[i], sacc[j0 + jj], 0, 0, 0, 127, 0, 127);
                }
#pragma unroll
                for (int jj = 0; jj < 2; ++jj) sacc[j0 + jj] *= qinv;
                if (T::kRopeSteps > 0 && hf == 1) {
#pragma unroll
                    for (int st = 0; st < T::kRopeSteps; ++st)
#pragma unroll
                        for (int jj = 0; jj < 2; ++jj) {
                            const u32x2 raw = *reinterpret_cast<const u32x2 *>(
                                kbuf + tile_pos<BK>(16 * (j0 + jj) + col, 512 + 32 * st + 8 * grp));
                            sacc[j0 + jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                fp8x8_to_bf16x8(raw.x, raw.y), qrope[st], sacc[j0 + jj], 0, 0, 0);
                        }
                }
            }
#pragma unroll
            for (int j = 0; j < NSB; ++j) sx[(wave * NSB + j) * 64 + lane] = sacc[j];
        }
        __syncthreads();
        if (!pair_active) continue;
#pragma unroll
        for (int j = 0; j < NSB; ++j) sacc[j] += sx[((wave ^ 2) * NSB + j) * 64 + lane];

        // Online softmax in base 2 over this tile (identical in both waves of the pair).
        const int tb = k0 + it * BK;
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < NSB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = tb + 16 * j + 4 * grp + i;
                const float sv = k < row_end ? sacc[j][i] * a.score_scale : kNegInf;
                sacc[j][i] = sv;
                mx = fmaxf(mx, sv);
            }
        mx = fmaxf(mx, xor_shuffle(mx, 16));
        mx = fmaxf(mx, xor_shuffle(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < NSB; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(sacc[j][i] - m_use);
                sacc[j][i] = p;
                psum += p;
            }
        psum += xor_shuffle(psum, 16);
        psum += xor_shuffle(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int v = 0; v < T::kVBlocks; ++v) oacc[v] *= alpha;
        }

        // O^T += V^T P^T, 32 keys per step.  Lane (s = 2k + h) of group g points the transposed
        // read at key 4g+k (k < 4) or 16+4g+k-4 (k >= 4), value bytes 8h..8h+7 of the block; the
        // read returns, for value column `col`, those 8 keys in k order -- the keys P^T holds in
        // slots 0..7 of lane group g.
        const int sl = lane & 15;
        const int kk = sl >> 1;
        const int key_in_step = kk < 4 ? 4 * grp + kk : 12 + 4 * grp + kk;
        const int vbase = hf * T::kHalfV + 8 * (sl & 1);
#pragma unroll
        for (int kb = 0; kb < T::kPvSteps; ++kb) {
            bf16x8 pf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pf[i] = static_cast<__bf16>(sacc[2 * kb][i]);
                pf[4 + i] = static_cast<__bf16>(sacc[2 * kb + 1][i]);
            }
            const int vkey = 32 * kb + key_in_step;
#pragma unroll
            for (int v = 0; v < T::kVBlocks; ++v) {
                const int2v raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) int2v *)(kbuf + tile_pos<BK>(vkey, vbase + 16 * v)));
                oacc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    fp8x8_to_bf16x8(uint32_t(raw.x), uint32_t(raw.y)), pf, oacc[v], 0, 0, 0);
            }
        }
    }

    if (!row_ok) return;
    // Lane holds O^T[hf*DV/2 + 16v + 4grp + i][col]: four consecutive values of its row.
    const int64_t row = int64_t(b) * a.rows_per_req + r_in;
    const float inv = l_run > 0.f ? a.out_scale / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    const int c0 = hf * T::kHalfV + 4 * grp;
    if (DIRECT) {
        uint16_t *o = a.out + row * DV + c0;
#pragma unroll
        for (int v = 0; v < T::kVBlocks; ++v)
            *reinterpret_cast<uint2 *>(o + 16 * v) =
                make_uint2(pack_bf16x2(oacc[v][0] * inv, oacc[v][1] * inv),
                           pack_bf16x2(oacc[v][2] * inv, oacc[v][3] * inv));
        if (hf == 0 && grp == 0 && a.lse2_out) a.lse2_out[row] = lse2;
    } else {
        float *o = a.part_o + (row * a.np + part) * DV + c0;
#pragma unroll
        for (int v = 0; v < T::kVBlocks; ++v)
            *reinterpret_cast<f32x4 *>(o + 16 * v) = oacc[v] * inv;
        if (hf == 0 && grp == 0) a.part_lse2[row * a.np + part] = lse2;
    }
}

#undef GQA_LOAD_INDICES
#undef GQA_LOAD_ROWS

template <int BK, int DQK, int DV>
hipError_t launch_shape(const MlaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(256);
    if (direct)
        hipLaunchKernelGGL((mla_split_kernel<BK, DQK, DV, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((mla_split_kernel<BK, DQK, DV, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mla_split(const MlaSplitArgs &a, int block_k, int d_qk, int d_v, bool direct,
                            hipStream_t s) {
    if (d_qk == 576 && d_v == 512)
        return block_k == 32 ? launch_shape<32, 576, 512>(a, direct, s)
                             : launch_shape<64, 576, 512>(a, direct, s);
    if (d_qk == 512 && d_v == 448)
        return block_k == 32 ? launch_shape<32, 512, 448>(a, direct, s)
                             : launch_shape<64, 512, 448>(a, direct, s);
    return hipErrorInvalidValue;
}

}  // namespace gqa
