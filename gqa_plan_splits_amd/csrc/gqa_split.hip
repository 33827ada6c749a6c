// gqa_split.hip -- split kernel of grouped-query decode over bf16 K/V pages, gfx950.
//
// What it computes (moonmath-amd README, gfx950 "forward_paged": caches
// [pages, page_size, kv_heads, 128], kv_indptr counting pages per sequence, kv_page_indices;
// Modular MAX planner page, MHA-style bullet: one CTA per (kv head, request) per partition):
// for one kv head of one request and one partition of its tokens, the query rows of that
// head group (q_len x group <= 16 of them) attend the partition's tokens; the CTA writes each
// row's softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Layout of the work (one wave per CTA):
//   - QK^T on v_mfma_f32_16x16x32_bf16 as S^T = K Q^T: each lane loads 16-byte pieces of one
//     token's K row straight into the A-operand layout (token = lane % 16), so K never touches
//     LDS; the query rows fill the 16 B-operand columns (unused columns are zero).
//   - Online softmax in base 2 in the MFMA output layout (lane column = query row).
//   - PV on the vector ALU: this path reads 8 flop per byte and is HBM-bound, and each lane
//     owning 8 value columns lets V rows be read as plain coalesced 16-byte loads with no
//     transpose.  Probabilities pass through 2 KB of LDS.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

constexpr int kD = 128;

template <int BK, int NR, bool DIRECT>
__global__ void __launch_bounds__(64) gqa_split_kernel(const GqaSplitArgs a) {
    constexpr int NSB = BK / 16;       // 16-token score blocks per tile
    constexpr int TPL = BK / 4;        // tokens per lane in the PV pass (4 token groups)
    __shared__ float pbuf[BK][17];     // probabilities [token][row], padded
    __shared__ float rowbuf[3][16];    // alpha, m, l per row

    const int logical = xcd_logical_block(blockIdx.x, a.total_ctas);
    if (logical < 0) return;
    const int kvh = logical % a.Hkv;
    const int rest = logical / a.Hkv;
    const int part = rest % a.np;
    const int b = rest / a.np;

    const int lane = threadIdx.x, grp = lane >> 4, col = lane & 15;
    const int rows_cta = a.q_len * a.group;
    const int page_mask = (1 << a.page_shift) - 1;

    const int S = a.seq_lens[b];
    const int pbase = a.kv_indptr[b];
    const int chunk = ((S + a.np - 1) / a.np + BK - 1) / BK * BK;
    const int k0 = part * chunk;
    const int block_keys = max(0, S - a.q_len + (rows_cta - 1) / a.group + 1);
    const int k1 = min(block_keys, k0 + chunk);
    const int ntiles = k1 > k0 ? (k1 - k0 + BK - 1) / BK : 0;

    // Query row in MFMA column `col`.
    const bool row_ok = col < rows_cta;
    const int t = row_ok ? col / a.group : 0;
    const int head = kvh * a.group + (row_ok ? col - t * a.group : 0);
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;

    bf16x8 qf[4];  // B operand: row col, d = 32 s + 8 grp .. +7
    {
        const uint16_t *q = a.q + (int64_t(b) * a.q_len + t) * a.q_st_tok + int64_t(head) * a.q_st_head;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qf[s] = as_bf16x8(row_ok ? *reinterpret_cast<const uint4 *>(q + 32 * s + 8 * grp)
                                     : make_uint4(0, 0, 0, 0));
    }

    const size_t kv_head_off = size_t(kvh) * kD;
    auto row_ptr = [&](const uint16_t *cache, int token) -> const uint16_t * {
        const int page = a.page_indices[pbase + (token >> a.page_shift)];
        const int64_t tok_slot = (int64_t(page) << a.page_shift) | (token & page_mask);
        return cache + tok_slot * (int64_t(a.Hkv) * kD) + kv_head_off;
    };

    // Register tiles: K in A-operand layout (token 16 kb + col, d = 32 s + 8 grp) and V chunks
    // (token grp + 4 m, values 8 col .. 8 col + 7).
    uint4 kreg[NSB][4], vreg[TPL];
    auto load_tile = [&](int tile) {
        const int tb = k0 + tile * BK;
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
            const int tok = tb + 16 * j + col;
            const bool ok = tok < k1;
            const uint16_t *p = ok ? row_ptr(a.k_cache, tok) : nullptr;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kreg[j][s] = ok ? *reinterpret_cast<const uint4 *>(p + 32 * s + 8 * grp)
                                : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < TPL; ++m) {
            const int tok = tb + grp + 4 * m;
            vreg[m] = tok < k1 ? *reinterpret_cast<const uint4 *>(row_ptr(a.v_cache, tok) + 8 * col)
                               : make_uint4(0, 0, 0, 0);
        }
    };

    float m_run = kNegInf, l_run = 0.f;
    float o[NR][8];
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[n][e] = 0.f;

    if (ntiles > 0) load_tile(0);
    for (int it = 0; it < ntiles; ++it) {
        uint4 kcur[NSB][4], vcur[TPL];
#pragma unroll
        for (int j = 0; j < NSB; ++j)
#pragma unroll
            for (int s = 0; s < 4; ++s) kcur[j][s] = kreg[j][s];
#pragma unroll
        for (int m = 0; m < TPL; ++m) vcur[m] = vreg[m];
        if (it + 1 < ntiles) load_tile(it + 1);

        f32x4 sacc[NSB];
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
            sacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kcur[j][s]), qf[s], sacc[j], 0, 0, 0);
        }

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
                psum += p;
                pbuf[16 * j + 4 * grp + i][col] = p;
            }
        psum += xor_shuffle(psum, 16);
        psum += xor_shuffle(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (grp == 0) rowbuf[0][col] = alpha;
        __syncthreads();

#pragma unroll
        for (int n = 0; n < NR; ++n) {
            const float al = rowbuf[0][n];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[n][e] *= al;
        }
#pragma unroll
        for (int m = 0; m < TPL; ++m) {
            const int tok = grp + 4 * m;
            float v[8];
            v[0] = bf16_lo(vcur[m].x); v[1] = bf16_hi(vcur[m].x);
            v[2] = bf16_lo(vcur[m].y); v[3] = bf16_hi(vcur[m].y);
            v[4] = bf16_lo(vcur[m].z); v[5] = bf16_hi(vcur[m].z);
            v[6] = bf16_lo(vcur[m].w); v[7] = bf16_hi(vcur[m].w);
#pragma unroll
            for (int n = 0; n < NR; ++n) {
                const float p = pbuf[tok][n];
#pragma unroll
                for (int e = 0; e < 8; ++e) o[n][e] = fmaf(p, v[e], o[n][e]);
            }
        }
        __syncthreads();
    }

    // Sum the four token groups' partial outputs; lanes 0..15 then own value columns 8 col..+7.
#pragma unroll
    for (int n = 0; n < NR; ++n)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[n][e] += xor_shuffle(o[n][e], 16);
            o[n][e] += xor_shuffle(o[n][e], 32);
        }
    if (grp == 0) {
        rowbuf[1][col] = m_run;
        rowbuf[2][col] = l_run;
    }
    __syncthreads();
    if (grp != 0) return;
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        if (n >= rows_cta) continue;
        const int tn = n / a.group;
        const int hn = kvh * a.group + (n - tn * a.group);
        const int64_t row = (int64_t(b) * a.q_len + tn) * a.Hq + hn;
        const float l = rowbuf[2][n];
        const float inv = l > 0.f ? 1.f / l : 0.f;
        if (DIRECT) {
            uint4 w;
            w.x = pack_bf16x2(o[n][0] * inv, o[n][1] * inv);
            w.y = pack_bf16x2(o[n][2] * inv, o[n][3] * inv);
            w.z = pack_bf16x2(o[n][4] * inv, o[n][5] * inv);
            w.w = pack_bf16x2(o[n][6] * inv, o[n][7] * inv);
            *reinterpret_cast<uint4 *>(a.out + row * kD + 8 * col) = w;
            if (col == 0 && a.lse2_out) a.lse2_out[row] = l > 0.f ? rowbuf[1][n] + __log2f(l) : kNegInf;
        } else {
            float *dst = a.part_o + (row * a.np + part) * kD + 8 * col;
            *reinterpret_cast<f32x4 *>(dst) = f32x4{o[n][0] * inv, o[n][1] * inv, o[n][2] * inv, o[n][3] * inv};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{o[n][4] * inv, o[n][5] * inv, o[n][6] * inv, o[n][7] * inv};
            if (col == 0) a.part_lse2[row * a.np + part] = l > 0.f ? rowbuf[1][n] + __log2f(l) : kNegInf;
        }
    }
}

template <int BK, int NR>
hipError_t launch_shape(const GqaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(xcd_grid_size(a.total_ctas)), block(64);
    if (direct)
        hipLaunchKernelGGL((gqa_split_kernel<BK, NR, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gqa_split_kernel<BK, NR, false>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gqa_split(const GqaSplitArgs &a, int block_k, int rows_per_cta, bool direct,
                            hipStream_t s) {
    if (rows_per_cta <= 8)
        return block_k == 32 ? launch_shape<32, 8>(a, direct, s) : launch_shape<64, 8>(a, direct, s);
    return block_k == 32 ? launch_shape<32, 16>(a, direct, s) : launch_shape<64, 16>(a, direct, s);
}

}  // namespace gqa
