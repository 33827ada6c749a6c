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
    static constexpr int kHalfD = DQK / 2;             // QK contraction per wave
    static constexpr int kKSteps = kHalfD / 32;        // MFMA K-steps per wave (9 or 8)
    static constexpr int kPairs = kKSteps / 2;         // steps read as 16-byte pairs
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

// d offset (within the wave's half of the row) of k-step s, lane group g, slot 0: steps are read
// in pairs as 16 contiguous bytes; an odd last step uses the plain 8-byte layout.
template <int KSTEPS>
__device__ __forceinline__ int kstep_offset(int s, int g) {
    if (s < (KSTEPS & ~1)) return 64 * (s >> 1) + 16 * g + 8 * (s & 1);
    return 32 * s + 8 * g;
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

    // Q^T fragments (MFMA B operand) for this wave's half of the contraction.
    const int dbase = hf * T::kHalfD;
    bf16x8 qf[T::kKSteps];
    {
        const int64_t tok = int64_t(b) * a.q_len + t;
        const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(h) * a.q_st_head;
        const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(h) * a.qpe_st_head;
#pragma unroll
        for (int s = 0; s < T::kKSteps; ++s) {
            const int d = dbase + kstep_offset<T::kKSteps>(s, grp);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (row_ok)
                v = d < T::kDLat ? *reinterpret_cast<const uint4 *>(ql + d)
                                 : *reinterpret_cast<const uint4 *>(qp + (d - T::kDLat));
            qf[s] = as_bf16x8(v);
        }
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[T::kVBlocks];
#pragma unroll
    for (int v = 0; v < T::kVBlocks; ++v) oacc[v] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Gather: item i = tid + 256 u is chunk (i % kChunks) of tile key (i / kChunks).
    uint4 stg[IPT];
    int idx[IPT];
    auto load_indices = [&](int tile) {   // branch-free: clamp to a valid key, then mask
        const int tb = k0 + tile * BK;
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int item = min(tid + u * T::kThreads, T::kItems - 1);
            const int k = tb + item / T::kChunks;
            const int slot = a.kv_indices[base + min(k, k1 - 1)];
            idx[u] = (tid + u * T::kThreads < T::kItems && k < k1) ? slot : -1;
        }
    };
    auto load_rows = [&]() {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int item = tid + u * T::kThreads;
            const int64_t off = int64_t(idx[u] < 0 ? 0 : idx[u]) * a.kv_stride + 16 * (item % T::kChunks);
            const uint4 v = *reinterpret_cast<const uint4 *>(a.kv + off);
            stg[u] = idx[u] < 0 ? make_uint4(0, 0, 0, 0) : v;   // padding keys hold zeros
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int u = 0; u < IPT; ++u) {
            const int item = tid + u * T::kThreads;
            if (item < T::kItems)
                *reinterpret_cast<uint4 *>(kbuf + tile_pos<BK>(item / T::kChunks, 16 * (item % T::kChunks))) = stg[u];
        }
    };

    if (ntiles > 0) {
        load_indices(0);
        load_rows();
        if (ntiles > 1) load_indices(1);
    }

    for (int it = 0; it < ntiles; ++it) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (it + 1 < ntiles) {
            load_rows();
            if (it + 2 < ntiles) load_indices(it + 2);
        }

        // Partial S^T over this wave's half of the row: block j covers keys 16j..16j+15; lane
        // holds keys 16j+4grp+i of row col.
        f32x4 sacc[NSB];
        if (pair_active) {
#pragma unroll
            for (int j = 0; j < NSB; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < T::kPairs; ++p) {
#pragma unroll
                for (int j = 0; j < NSB; ++j) {
                    const uint4 raw = *reinterpret_cast<const uint4 *>(
                        kbuf + tile_pos<BK>(16 * j + col, dbase + 64 * p + 16 * grp));
                    sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw.x, raw.y),
                                                                      qf[2 * p], sacc[j], 0, 0, 0);
                    sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw.z, raw.w),
                                                                      qf[2 * p + 1], sacc[j], 0, 0, 0);
                }
            }
            if (T::kKSteps & 1) {
                constexpr int s = T::kKSteps - 1;
#pragma unroll
                for (int j = 0; j < NSB; ++j) {
                    const uint2 raw = *reinterpret_cast<const uint2 *>(
                        kbuf + tile_pos<BK>(16 * j + col, dbase + 32 * s + 8 * grp));
                    sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw.x, raw.y),
                                                                      qf[s], sacc[j], 0, 0, 0);
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
