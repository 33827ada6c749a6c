// mla_split.hip -- split kernel of absorbed MLA decode for gfx950.
//
// What it computes (moonmath-amd README, "MLA decode"; Modular MAX planner page, MLA-style
// bullet): every key row of the pool is one fused fp8 e4m3 row that serves as K (all DQK bytes)
// and as V (its first DV bytes), dequantized with one per-tensor kv_scale.  A CTA packs 32 query
// rows (BM = 32) of one request and walks one partition of that request's keys, writing the
// partition's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Layout of the work:
//   - 128 threads = 2 waves; wave w owns rows 16w..16w+15 of the CTA's 32.
//   - Keys are processed in tiles of BK (32 or 64).  All 128 threads gather a tile (16 bytes per
//     lane per load, slot ids read a tile ahead) into registers one tile ahead of the compute,
//     then write it to LDS twice: row-major (the QK^T operand) and transposed (the PV operand).
//   - QK^T and PV run on v_mfma_f32_16x16x32_bf16: the fp8 bytes are converted to bf16 exactly
//     as they are read from LDS; kv_scale is folded into the score scale and the output scale.
//   - Scores are S^T = K Q^T (rows = keys, columns = query rows), so each lane owns one query
//     row's column: the row max / sum take two cross-lane exchanges, and the output O^T = V^T P^T
//     has each lane's accumulators in a single query row, so the online-softmax rescale is a
//     per-lane multiply.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

template <int BK, int DQK, int DV>
struct MlaTile {
    static constexpr int kThreads = 128;
    static constexpr int kDLat = DQK - 64;            // latent width; V = first DV columns
    static constexpr int kKSteps = DQK / 32;          // MFMA K-steps over the key row
    static constexpr int kVBlocks = DV / 16;          // 16-wide blocks of the value width
    static constexpr int kSBlocks = BK / 16;          // 16-key score blocks per tile
    static constexpr int kPvSteps = BK / 32;          // 32-key PV steps per tile
    static constexpr int kKStride = DQK + 8;          // bytes per K row in LDS (8 * odd)
    static constexpr int kKeysPerThread = BK / 4;     // main gather: 32 chunks x 4 key groups
    static constexpr int kExtraChunks = (DQK - 512) / 16;               // chunks past 512 bytes
    static constexpr int kExtraPerThread = kExtraChunks * BK / kThreads;  // 0, 1 or 2
    static constexpr int kVChunks = DV / 16;          // 16-byte chunks that are also values
    static constexpr int kKBytes = BK * kKStride;
    static constexpr int kVBytes = DV * BK;
    static constexpr int kLdsBytes = kKBytes + kVBytes;
    static_assert(DQK == 576 || DQK == 512, "row width");
    static_assert(DV % 16 == 0 && DV <= kDLat, "value width");
    static_assert(BK == 32 || BK == 64, "tile");
    static_assert(kExtraChunks * BK % kThreads == 0, "extra chunks per thread");
};

// Position of a key inside the transposed V tile.  The PV MFMA consumes 32 keys per step; lane
// group g (lanes 16g..16g+15) supplies k-slots 8g..8g+7, which hold keys 4g..4g+3 (from the
// first 16-key score block) and 16+4g..16+4g+3 (from the second) -- exactly the keys that lane
// group owns in the score output layout.  key_of_position inverts that order.
__device__ __forceinline__ int key_of_position(int p) {
    const int r = p & 31;
    return (p & ~31) + ((r >> 2) & 1) * 16 + (r >> 3) * 4 + (r & 3);
}

// Byte offset of (value block vb, PV step kb, lane group grp, row j of the block) in the
// transposed V tile.  Each (vb, kb, grp) owns 128 contiguous bytes = 16 slots of 8 keys; row j
// sits in slot (j + vb) % 16.  Readers (16 lanes = 16 rows) hit 16 distinct slots; writers
// (16 lanes = 16 value blocks, same row) also hit 16 distinct slots: both conflict-free.
template <int NPV>
__device__ __forceinline__ int vt_offset(int vb, int kb, int grp, int j) {
    return ((((vb * NPV + kb) << 2) + grp) * 16 + ((j + vb) & 15)) * 8;
}

template <int BK, int DQK, int DV, bool DIRECT>
__global__ void __launch_bounds__(128) mla_split_kernel(const MlaSplitArgs a) {
    using T = MlaTile<BK, DQK, DV>;
    constexpr int KPT = T::kKeysPerThread;
    constexpr int XPT = T::kExtraPerThread > 0 ? T::kExtraPerThread : 1;
    constexpr int NPV = T::kPvSteps;

    __shared__ __attribute__((aligned(16))) uint8_t lds[T::kLdsBytes];
    uint8_t *const kbuf = lds;
    uint8_t *const vbuf = lds + T::kKBytes;

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

    // The query row whose column this lane holds.
    const int r_in = row_lo + wave * 16 + col;
    const bool row_ok = r_in < a.rows_per_req;
    const int t = row_ok ? r_in / a.H : 0;
    const int h = row_ok ? r_in - t * a.H : 0;
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;
    const bool wave_active = row_lo + wave * 16 < a.rows_per_req;

    // Q^T fragments (MFMA B operand): lane holds query row `col`, d = 32 s + 8 grp .. +7.
    bf16x8 qf[T::kKSteps];
    {
        const int64_t tok = int64_t(b) * a.q_len + t;
        const uint16_t *ql = a.q + tok * a.q_st_tok + int64_t(h) * a.q_st_head;
        const uint16_t *qp = a.q_pe + tok * a.qpe_st_tok + int64_t(h) * a.qpe_st_head;
#pragma unroll
        for (int s = 0; s < T::kKSteps; ++s) {
            const int d = 32 * s + 8 * grp;
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

    // Gather mapping: thread (c, kg) moves 16-byte chunk c of the first 512 bytes of the KPT keys
    // at tile positions kg*KPT .. kg*KPT+KPT-1, plus XPT chunks past 512 bytes (576-wide rows).
    const int c = tid & 31, kg = tid >> 5;
    uint4 st_main[KPT];
    uint4 st_extra[XPT];
    int idx_main[KPT];
    int idx_extra[XPT];

    auto load_indices = [&](int tile) {
        const int tb = k0 + tile * BK;
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            const int k = tb + key_of_position(kg * KPT + u);
            idx_main[u] = k < k1 ? a.kv_indices[base + k] : -1;
        }
        if (T::kExtraPerThread > 0) {
#pragma unroll
            for (int x = 0; x < XPT; ++x) {
                const int item = tid + x * T::kThreads;
                const int k = tb + item / T::kExtraChunks;
                idx_extra[x] = k < k1 ? a.kv_indices[base + k] : -1;
            }
        }
    };
    auto load_rows = [&]() {
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            st_main[u] = make_uint4(0, 0, 0, 0);
            if (idx_main[u] >= 0)
                st_main[u] = *reinterpret_cast<const uint4 *>(
                    a.kv + int64_t(idx_main[u]) * a.kv_stride + 16 * c);
        }
        if (T::kExtraPerThread > 0) {
#pragma unroll
            for (int x = 0; x < XPT; ++x) {
                const int item = tid + x * T::kThreads;
                const int ch = 32 + item % T::kExtraChunks;
                st_extra[x] = make_uint4(0, 0, 0, 0);
                if (idx_extra[x] >= 0)
                    st_extra[x] = *reinterpret_cast<const uint4 *>(
                        a.kv + int64_t(idx_extra[x]) * a.kv_stride + 16 * ch);
            }
        }
    };
    auto store_tile = [&]() {
        // K, row-major in natural key order (two 8-byte writes: rows are 8-byte aligned).
#pragma unroll
        for (int u = 0; u < KPT; ++u) {
            uint2 *dst = reinterpret_cast<uint2 *>(kbuf + key_of_position(kg * KPT + u) * T::kKStride + 16 * c);
            dst[0] = make_uint2(st_main[u].x, st_main[u].y);
            dst[1] = make_uint2(st_main[u].z, st_main[u].w);
        }
        if (T::kExtraPerThread > 0) {
#pragma unroll
            for (int x = 0; x < XPT; ++x) {
                const int item = tid + x * T::kThreads;
                const int key = item / T::kExtraChunks;
                const int ch = 32 + item % T::kExtraChunks;
                uint2 *dst = reinterpret_cast<uint2 *>(kbuf + key * T::kKStride + 16 * ch);
                dst[0] = make_uint2(st_extra[x].x, st_extra[x].y);
                dst[1] = make_uint2(st_extra[x].z, st_extra[x].w);
            }
        }
        // V^T: 4x4 byte transposes turn (4 keys x 16 values) into (16 values x 4 keys).
        if (c < T::kVChunks) {
#pragma unroll
            for (int pg = 0; pg < KPT / 8; ++pg) {
                const int p0 = kg * KPT + 8 * pg;
                const int kb = p0 >> 5, g8 = (p0 & 31) >> 3;
                uint32_t y[2][16];
#pragma unroll
                for (int qq = 0; qq < 2; ++qq) {
                    const uint4 *x = st_main + 8 * pg + 4 * qq;
                    transpose4x4_bytes(x[0].x, x[1].x, x[2].x, x[3].x, y[qq][0], y[qq][1], y[qq][2], y[qq][3]);
                    transpose4x4_bytes(x[0].y, x[1].y, x[2].y, x[3].y, y[qq][4], y[qq][5], y[qq][6], y[qq][7]);
                    transpose4x4_bytes(x[0].z, x[1].z, x[2].z, x[3].z, y[qq][8], y[qq][9], y[qq][10], y[qq][11]);
                    transpose4x4_bytes(x[0].w, x[1].w, x[2].w, x[3].w, y[qq][12], y[qq][13], y[qq][14], y[qq][15]);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    *reinterpret_cast<uint2 *>(vbuf + vt_offset<NPV>(c, kb, g8, j)) =
                        make_uint2(y[0][j], y[1][j]);
            }
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
        if (!wave_active) continue;

        // S^T = K Q^T: block j covers keys 16j..16j+15; lane holds keys 16j+4grp+i of row col.
        f32x4 sacc[T::kSBlocks];
#pragma unroll
        for (int j = 0; j < T::kSBlocks; ++j) sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < T::kKSteps; ++s) {
#pragma unroll
            for (int j = 0; j < T::kSBlocks; ++j) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(
                    kbuf + (16 * j + col) * T::kKStride + 32 * s + 8 * grp);
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw.x, raw.y),
                                                                  qf[s], sacc[j], 0, 0, 0);
            }
        }

        // Online softmax in base 2 over this tile.
        const int tb = k0 + it * BK;
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < T::kSBlocks; ++j)
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
        for (int j = 0; j < T::kSBlocks; ++j)
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
#pragma unroll
        for (int v = 0; v < T::kVBlocks; ++v) oacc[v] *= alpha;

        // O^T += V^T P^T, 32 keys per step.
#pragma unroll
        for (int kb = 0; kb < NPV; ++kb) {
            bf16x8 pf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pf[i] = static_cast<__bf16>(sacc[2 * kb][i]);
                pf[4 + i] = static_cast<__bf16>(sacc[2 * kb + 1][i]);
            }
#pragma unroll
            for (int v = 0; v < T::kVBlocks; ++v) {
                const uint2 raw = *reinterpret_cast<const uint2 *>(vbuf + vt_offset<NPV>(v, kb, grp, col));
                oacc[v] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fp8x8_to_bf16x8(raw.x, raw.y), pf,
                                                                  oacc[v], 0, 0, 0);
            }
        }
    }

    if (!row_ok) return;
    // Lane holds O^T[16v + 4grp + i][col]: four consecutive values of its row.
    const int64_t row = int64_t(b) * a.rows_per_req + r_in;
    const float inv = l_run > 0.f ? a.out_scale / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    if (DIRECT) {
        uint16_t *o = a.out + row * DV + 4 * grp;
#pragma unroll
        for (int v = 0; v < T::kVBlocks; ++v)
            *reinterpret_cast<uint2 *>(o + 16 * v) =
                make_uint2(pack_bf16x2(oacc[v][0] * inv, oacc[v][1] * inv),
                           pack_bf16x2(oacc[v][2] * inv, oacc[v][3] * inv));
        if (grp == 0 && a.lse2_out) a.lse2_out[row] = lse2;
    } else {
        float *o = a.part_o + (row * a.np + part) * DV + 4 * grp;
#pragma unroll
        for (int v = 0; v < T::kVBlocks; ++v)
            *reinterpret_cast<f32x4 *>(o + 16 * v) = oacc[v] * inv;
        if (grp == 0) a.part_lse2[row * a.np + part] = lse2;
    }
}

template <int BK, int DQK, int DV>
hipError_t launch_shape(const MlaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(128);
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
