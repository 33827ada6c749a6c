// splitk_reduce.hip -- fp32 base-2 LSE merge of up to 256 partitions, gfx950.
//
// What it computes (Modular MAX planner page, "AMD reducer constraint": the reducer merges up
// to parts_per_lane x WARP_SIZE partitions, 4 x 64 = 256): for each row,
//   lse2 = log2(sum_i 2^lse2_i),   o = sum_i 2^(lse2_i - lse2) * o_i,
// with the weights summed in partition order 0..np-1 (a fixed association, so the result is
// deterministic).  Output rounded to bf16, nearest even (moonmath-amd README, gfx950 RTNE).
//
// One wave64 per row: each lane holds up to four partition LSEs, the row max and the weight
// sum are two butterfly reductions, and the weights are shared through LDS while every lane
// streams 16-byte pieces of the partial outputs.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

constexpr int kWavesPerBlock = 4;

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

__global__ void __launch_bounds__(256) splitk_reduce_kernel(const ReduceArgs a) {
    __shared__ float wbuf[kWavesPerBlock][256];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int64_t row = int64_t(blockIdx.x) * kWavesPerBlock + w;
    if (row >= a.rows) return;   // whole waves exit together: no block barrier is used below

    const float *lp = a.part_lse2 + row * a.np;
    float l4[4];
    float mx = kNegInf;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = lane + 64 * k;
        l4[k] = p < a.np ? lp[p] : kNegInf;
        mx = fmaxf(mx, l4[k]);
    }
    mx = wave_max(mx);
    const int nvec = a.dv >> 2;
    uint16_t *out = a.out + row * a.dv;
    if (mx == kNegInf) {   // no partition saw a key: the row is 0 with lse2 = -inf
        for (int v = lane; v < nvec; v += 64)
            *reinterpret_cast<uint2 *>(out + 4 * v) = make_uint2(0, 0);
        if (lane == 0 && a.lse2_out) a.lse2_out[row] = kNegInf;
        return;
    }
    float wsum = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = lane + 64 * k;
        const float wgt = fast_exp2(l4[k] - mx);   // -inf -> 0
        if (p < a.np) wbuf[w][p] = wgt;
        wsum += wgt;
    }
    wsum = wave_sum(wsum);
    const float inv = 1.f / wsum;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const float *po = a.part_o + row * int64_t(a.np) * a.dv;
    for (int v = lane; v < nvec; v += 64) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int p = 0; p < a.np; ++p) {
            const float wgt = wbuf[w][p];
            if (wgt == 0.f) continue;   // empty partition: its output is not read
            acc += wgt * *reinterpret_cast<const f32x4 *>(po + int64_t(p) * a.dv + 4 * v);
        }
        acc *= inv;
        *reinterpret_cast<uint2 *>(out + 4 * v) =
            make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
    }
    if (lane == 0 && a.lse2_out) a.lse2_out[row] = mx + __log2f(wsum);
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
    const int64_t blocks = (a.rows + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3(unsigned(blocks)), dim3(64 * kWavesPerBlock), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fp8_to_bf16(const uint8_t *in, int64_t n, uint16_t *out, hipStream_t s) {
    const int64_t threads = (n + 7) / 8;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(fp8_to_bf16_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, in, n, out);
    return hipGetLastError();
}

}  // namespace gqa
