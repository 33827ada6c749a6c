// plan_device.hip -- the device-side planner of length-proportional partitions: the plan is
// made from the lengths in device memory, with no host synchronization, so a captured decode
// replays with new lengths and re-plans each time ([MM] "VarlenPlan": planning on the GPU from
// device-side lengths; the length-proportional split is this library's reading).
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanCached = 8192;   // requests whose key counts the search reads from LDS

// Keys of request b (negative counts as none), held to kMaxKeys = 2^31 - 64, a multiple of
// block_k: every chunk below is then a multiple of block_k of at most kMaxKeys, so it fits an
// int32 and n + c - 1 fits 32 bits.
constexpr int64_t kMaxKeys = (int64_t(1) << 31) - 64;
__device__ __forceinline__ uint32_t keys_in_memory(const PlanArgs &a, int b) {
    int64_t n = a.seq_lens[b];
    if (a.extra_indptr) n += int64_t(a.extra_indptr[b + 1]) - a.extra_indptr[b];
    return uint32_t(min(max(n, int64_t(0)), kMaxKeys));
}

// Slots of a request with n keys under the common chunk c, and the chunk it uses (n, c <=
// kMaxKeys, so n + c - 1 fits 32 bits, and the chunk stays at most kMaxKeys).
__device__ __forceinline__ void slots_of(const PlanArgs &a, uint32_t n, uint32_t c, int *slots,
                                         int *chunk) {
    uint32_t k = (n + c - 1) / c;
    if (k > uint32_t(a.cap)) {
        const uint32_t bk = uint32_t(a.block_k), per = (n + a.cap - 1) / uint32_t(a.cap);
        c = (per + bk - 1) / bk * bk;
        k = (n + c - 1) / c;
    }
    *slots = int(k);
    *chunk = int(c);
}

// Sum over the workgroup of v (every thread gets it); `slot` is the caller's LDS scratch.
__device__ __forceinline__ int64_t block_sum(int64_t v, int64_t *slot) {
    for (int m = 32; m; m >>= 1) v += __shfl_xor(v, m, 64);
    __syncthreads();   // the previous use of slot is over
    if ((threadIdx.x & 63) == 0) slot[threadIdx.x >> 6] = v;
    __syncthreads();
    int64_t t = 0;
    for (int w = 0; w < kPlanWaves; ++w) t += slot[w];
    return t;
}

__global__ void __launch_bounds__(kPlanThreads) plan_proportional_kernel(const PlanArgs a) {
    __shared__ int64_t wave_sum[kPlanWaves];
    __shared__ int32_t wave_scan[kPlanWaves];
    __shared__ uint32_t cached[kPlanCached];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool use_lds = a.batch <= kPlanCached;
    for (int b = threadIdx.x; use_lds && b < a.batch; b += kPlanThreads)
        cached[b] = keys_in_memory(a, b);
    __syncthreads();
    auto keys_of = [&](int b) -> uint32_t { return use_lds ? cached[b] : keys_in_memory(a, b); };

    // The common partition length: the smallest multiple of block_k whose slots, summed over
    // the batch, fit the budget (slot counts only fall as it grows, so a binary search finds it;
    // at the longest request rounded up every request takes at most one slot).
    int64_t longest = 0;
    for (int b = threadIdx.x; b < a.batch; b += kPlanThreads) longest = max(longest, int64_t(keys_of(b)));
    for (int m = 32; m; m >>= 1) longest = max(longest, __shfl_xor(longest, m, 64));
    if (lane == 0) wave_sum[wave] = longest;
    __syncthreads();
    for (int w = 0; w < kPlanWaves; ++w) longest = max(longest, wave_sum[w]);
    int64_t lo = 1, hi = max(int64_t(1), (longest + a.block_k - 1) / a.block_k);
    while (lo < hi) {   // workgroup-uniform
        const int64_t mid = (lo + hi) / 2;
        int64_t n = 0;
        for (int b = threadIdx.x; b < a.batch; b += kPlanThreads) {
            int slots, chunk;
            slots_of(a, keys_of(b), uint32_t(mid * a.block_k), &slots, &chunk);
            n += slots;
        }
        if (block_sum(n, wave_sum) <= a.budget) hi = mid;
        else lo = mid + 1;
    }
    const int64_t common = lo * a.block_k;

    // part_start: exclusive prefix sum of the slot counts, 256 requests at a time
    if (threadIdx.x == 0) a.part_start[0] = 0;
    int carry = 0;
    for (int b0 = 0; b0 < a.batch; b0 += kPlanThreads) {
        const int b = b0 + threadIdx.x;
        int slots = 0, chunk = 0;
        if (b < a.batch) slots_of(a, keys_of(b), uint32_t(common), &slots, &chunk);
        int x = slots;   // inclusive scan within the wave
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        if (lane == 63) wave_scan[wave] = x;
        __syncthreads();
        int before = carry, all = carry;
        for (int w = 0; w < kPlanWaves; ++w) {
            if (w < wave) before += wave_scan[w];
            all += wave_scan[w];
        }
        if (b < a.batch) {
            a.part_start[b + 1] = before + x;
            a.part_chunk[b] = chunk;
        }
        carry = all;
        __syncthreads();   // wave_scan is rewritten by the next round
    }
}

}  // namespace

hipError_t launch_plan_proportional(const PlanArgs &a, hipStream_t s) {
    if (a.batch < 1 || a.budget < 1 || a.cap < 1 || a.block_k < 1 || !a.part_start || !a.part_chunk)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(plan_proportional_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace gqa
