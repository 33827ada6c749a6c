// splitk_reduce.hip -- fp32 base-2 LSE merge of up to 256 partitions, gfx950.
//
// What it computes (Modular MAX planner page, "AMD reducer constraint": the reducer merges up
// to parts_per_lane x WARP_SIZE partitions, 4 x 64 = 256; the same merge combines the ranks of
// decode context parallelism, moonmath-amd README "MLA decode"): for each row,
//   lse2 = log2(sum_i 2^lse2_i),   o = sum_i 2^(lse2_i - lse2) * o_i,
// in fp32 with a fixed association (so the result is deterministic).  Output rounded to bf16,
// nearest even (moonmath-amd README, gfx950 RTNE), or kept in fp32 for a caller that merges
// further (a context-parallel rank).
//
// Layout of the work, per (row, column chunk) item; four waves per block.  A chunk is 256
// columns (64 lanes x 4) when rows are few, the whole row when there are enough of them.
//   - Many items (or few partitions): one wave per item.
//   - Few items and many partitions (a small batch split 64 ways): one block per item, wave w
//     summing partitions w, w + 4, .., so that a few long rows still spread over the chip; the
//     four waves' sums are added in wave order through LDS.
// Every wave computes the row's LSE maximum and weights itself (each lane holds up to four
// partition LSEs; two butterfly reductions) and keeps them in its own LDS slice; each lane sums
// its four columns over its partitions four at a time (four loads in flight, one accumulator
// each).  The association is fixed for a given shape, so the result is deterministic.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxBlocks = 1 << 20;   // larger inputs loop over their items

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, xor_shuffle(v, m));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += xor_shuffle(v, m);
    return v;
}

__device__ __forceinline__ f32x4 load4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// Four output values: bf16 rounded to nearest even, or fp32.
template <bool F32OUT>
__device__ __forceinline__ void store4(const ReduceArgs &a, int64_t row, int c4, f32x4 v) {
    if (F32OUT)
        *reinterpret_cast<f32x4 *>(a.out_f32 + row * a.dv + 4 * c4) = v;
    else
        *reinterpret_cast<uint2 *>(a.out + row * a.dv + 4 * c4) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// SPLIT: the block's four waves share one item and split its partitions (stride 4, first w);
// otherwise wave w of block x owns item 4 x + w and every partition (stride 1).
template <bool SPLIT, bool F32OUT>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const ReduceArgs a, int chunks, int chunk_vec) {
    __shared__ float wbuf[kWaves][256];
    __shared__ f32x4 sums[kWaves - 1][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int nvec = a.dv >> 2;
    const int64_t items = a.rows * chunks;
    const int64_t step = SPLIT ? int64_t(gridDim.x) : int64_t(gridDim.x) * kWaves;
    const int pstep = SPLIT ? kWaves : 1;

    for (int64_t item = SPLIT ? blockIdx.x : int64_t(blockIdx.x) * kWaves + w; item < items; item += step) {
        const int64_t row = item / chunks;
        const int chunk = int(item - row * chunks);
        const int c_end = min(nvec, (chunk + 1) * chunk_vec);
        const bool lead = !SPLIT || w == 0;   // the wave that writes the item's output

        // the row's partitions: np of them at row * o_row (l_row), or with a plan the slots of
        // the row's request, slot-major
        int np = a.np;
        int64_t obase = row * a.o_row, lbase = row * a.l_row;
        if (a.part_start) {
            const int64_t b = row / a.rows_per_req, r = row - b * a.rows_per_req;
            const int s0 = a.part_start[b];
            np = a.part_start[b + 1] - s0;
            lbase = int64_t(s0) * a.rows_per_req + r;
            obase = lbase * a.dv;
        }
        const float *lp = a.part_lse2 + lbase;
        float l4[4];
        float mx = kNegInf;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int p = lane + 64 * k;
            l4[k] = p < np ? lp[p * a.l_part] : kNegInf;
            mx = fmaxf(mx, l4[k]);
        }
        mx = wave_max(mx);   // with SPLIT identical in the four waves: the branch is block-uniform
        if (mx == kNegInf) {   // no partition saw a key: the row is 0 with lse2 = -inf
            if (lead)
                for (int c4 = chunk * chunk_vec + lane; c4 < c_end; c4 += 64)
                    store4<F32OUT>(a, row, c4, f32x4{0.f, 0.f, 0.f, 0.f});
            if (lead && lane == 0 && chunk == 0 && a.lse2_out) a.lse2_out[row] = kNegInf;
            continue;
        }
        float wsum = 0.f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int p = lane + 64 * k;
            const float wgt = fast_exp2(l4[k] - mx);   // -inf -> 0
            if (p < np) wbuf[w][p] = wgt;
            wsum += wgt;
        }
        wsum = wave_sum(wsum);
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // Lane columns 4 c4 .. 4 c4 + 3.  Four partitions per iteration, each into its own
        // accumulator.  A partition without weight contributes nothing, whatever its output holds.
        // (With SPLIT a chunk is one pass of 64 lanes, so every wave reaches the barriers once.)
        const float inv = 1.f / wsum;
        for (int base = chunk * chunk_vec; base < c_end; base += 64) {
            const int c4 = base + lane;
            const bool col_ok = c4 < c_end;
            f32x4 acc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (col_ok) {
                const float *po = a.part_o + obase + 4 * c4;
                int p = SPLIT ? w : 0;
                for (; p + 3 * pstep < np; p += 4 * pstep) {
                    // weights are the row's, the same in every lane: a partition without weight
                    // is not loaded at all
                    f32x4 x[4];
                    float wg[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        wg[j] = wbuf[w][p + pstep * j];
                        x[j] = wg[j] != 0.f ? load4(po + int64_t(p + pstep * j) * a.o_part)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (wg[j] != 0.f) acc[j] += wg[j] * x[j];
                }
#pragma unroll
                for (int j = 0; j < 3; ++j) {   // at most three left
                    const int q = p + pstep * j;
                    if (q < np) {
                        const float wgt = wbuf[w][q];
                        if (wgt != 0.f) acc[j] += wgt * load4(po + int64_t(q) * a.o_part);
                    }
                }
            }
            f32x4 tot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
            if (SPLIT) {
                if (w > 0) sums[w - 1][lane] = tot;
                __syncthreads();
                if (w == 0) tot = ((tot + sums[0][lane]) + sums[1][lane]) + sums[2][lane];
                __syncthreads();   // sums are reused by the next item
            }
            if (lead && col_ok) store4<F32OUT>(a, row, c4, tot * inv);
        }
        if (lead && lane == 0 && chunk == 0 && a.lse2_out) a.lse2_out[row] = mx + __log2f(wsum);
    }
}

__global__ void __launch_bounds__(256) fp8_to_bf16_kernel(const uint8_t *in, int64_t n, uint16_t *out) {
    const int64_t i = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * 8;
    if (i + 8 <= n) {
        const uint2 raw = *reinterpret_cast<const uint2 *>(in + i);
        *reinterpret_cast<bf16x8 *>(out + i) = fp8x8_to_bf16x8(raw.x, raw.y);
    } else {
        for (int64_t j = i; j < n; ++j) {
            const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(uint32_t(in[j]), 1.0f, false);
            out[j] = __builtin_bit_cast(uint16_t, r.x);
        }
    }
}

}  // namespace

hipError_t launch_splitk_reduce(const ReduceArgs &a, hipStream_t s) {
    const int nvec = a.dv >> 2;
    const int c256 = (nvec + 63) / 64;   // 256-column chunks per row
    // Whole rows per wave once there are enough rows to fill the chip; otherwise 256-column
    // chunks, and the partitions of one chunk split over four waves when the chunks alone would
    // leave the chip mostly idle and there are enough partitions to share.
    const bool whole = a.rows >= 4096;
    const int chunks = whole ? 1 : c256;
    const int chunk_vec = whole ? 64 * c256 : 64;
    const int64_t items = a.rows * chunks;
    const bool split = !whole && items < 1024 && a.np >= 8;
    const int64_t need = split ? items : (items + kWaves - 1) / kWaves;
    const dim3 grid(unsigned(need < kMaxBlocks ? need : kMaxBlocks)), block(64 * kWaves);
    const bool f32 = a.out_f32 != nullptr;
    if (split && f32)
        hipLaunchKernelGGL((splitk_reduce_kernel<true, true>), grid, block, 0, s, a, chunks, chunk_vec);
    else if (split)
        hipLaunchKernelGGL((splitk_reduce_kernel<true, false>), grid, block, 0, s, a, chunks, chunk_vec);
    else if (f32)
        hipLaunchKernelGGL((splitk_reduce_kernel<false, true>), grid, block, 0, s, a, chunks, chunk_vec);
    else
        hipLaunchKernelGGL((splitk_reduce_kernel<false, false>), grid, block, 0, s, a, chunks, chunk_vec);
    return hipGetLastError();
}

hipError_t launch_fp8_to_bf16(const uint8_t *in, int64_t n, uint16_t *out, hipStream_t s) {
    const int64_t threads = (n + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, in, n, out);
    return hipGetLastError();
}

}  // namespace gqa
