// ceiling.hip -- data-movement ceilings for the benchmark: how fast this GPU moves bytes from HBM
// into LDS with the copy instruction the split kernels use (global_load_lds_dwordx4, non-temporal),
//   - as a plain stream of contiguous bytes, and
//   - as a gather of rows at listed slots, in the MLA split kernel's own copy pattern (each copy
//     instruction moves one 128-byte line of 8 rows; 64-byte rope tails 16 rows at a time),
//   - and as the same gather with each copy instruction moving the first 512 bytes of two rows
//     (whole-row requests; the rope tails as before),
// with no arithmetic.  The bytes land in LDS and are overwritten; nothing is written to memory.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/gqa_splits.h"
#include "kernels.hpp"

namespace gqa {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void copy16_nt(const void *g, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}

constexpr int kStreamThreads = 256;   // 4 waves, each with an 8-slot ring of 1 KiB
constexpr int kRing = 8;

// CTA c streams bytes [c * per_cta, (c + 1) * per_cta) of src (per_cta a multiple of 4 KiB); wave w
// takes every fourth KiB, 1 KiB per copy instruction, at most kRing copies in flight.
__global__ void __launch_bounds__(kStreamThreads) stream_read_kernel(const uint8_t *src, int64_t per_cta) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kRing * 1024];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint8_t *base = src + int64_t(blockIdx.x) * per_cta;
    const uint32_t ring = uint32_t(reinterpret_cast<uintptr_t>(lds)) + wave * kRing * 1024;
    const int64_t n = per_cta >> 10;
    int slot = 0;
    for (int64_t k = wave; k < n; k += 4) {
        copy16_nt(base + (k << 10) + 16 * lane, ring + slot * 1024);
        slot = (slot + 1) & (kRing - 1);
        asm volatile("s_waitcnt vmcnt(7)" ::: "memory");
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Rows of row_bytes (576 or 512) at the slots idx[0 .. n) (n a multiple of 64).  Wave w of CTA c
// takes the 64-row groups g = 4 c + w, 4 c + w + 4 * grid, ...; per group it issues the MLA split
// kernel's copies of one tile: for each line v (0..3), 8 instructions of 8 rows x 128 bytes (lane
// L: row 8 (L >> 3) + i, 16 bytes at 128 v + 16 (L & 7)); WHOLE: 32 instructions of 2 rows x 512
// bytes (lane L: row 2 i + (L >> 5), 16 bytes at 16 (L & 31)); and for 576-byte rows four instructions
// of 16 rope tails.  The group's slot ids come two groups ahead into a 4-slot LDS ring
// (global_load_lds_dword), waited for with explicit counts like the copies; all copies of a wave
// land in one 33 KiB area, overwritten (the bytes are not used).
constexpr int kGatherThreads = 256;
constexpr int kGatherArea = 33 * 1024;

__device__ __forceinline__ void copy4_nt(const int32_t *g, uint32_t m0) {
    asm volatile("global_load_lds_dword %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}

template <bool WHOLE>
__global__ void __launch_bounds__(kGatherThreads) gather_rows_kernel(const uint8_t *pool, int64_t row_bytes,
                                                                     const int32_t *idx, int64_t n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * kGatherArea + 4 * 4 * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int jgrp = lane >> 3;
    const bool tail = row_bytes > 512;
    const uint32_t area = uint32_t(reinterpret_cast<uintptr_t>(lds)) + wave * kGatherArea;
    uint8_t *const id_ring_p = lds + 4 * kGatherArea + wave * 4 * 256;
    const uint32_t id_ring = uint32_t(reinterpret_cast<uintptr_t>(id_ring_p));
    const int64_t groups = n >> 6;
    const int64_t first = int64_t(blockIdx.x) * 4 + wave, step = int64_t(gridDim.x) * 4;
    const int per_group = 32 + (tail ? 4 : 0);   // copy instructions per group
    auto load_ids = [&](int64_t k) {           // the k-th group of this wave
        const int64_t grp = first + k * step;
        if (grp < groups) copy4_nt(idx + (grp << 6) + lane, id_ring + (k & 3) * 256);
    };
    load_ids(0);
    load_ids(1);
    for (int64_t k = 0; first + k * step < groups; ++k) {
        // ids(k) landed: issued after them are copies(k - 1) and ids(k + 1) (in the first
        // iteration only ids(1))
        if (k == 0)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else if (per_group == 32)
            asm volatile("s_waitcnt vmcnt(33)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(37)" ::: "memory");
        const int32_t *ids = reinterpret_cast<const int32_t *>(id_ring_p + (k & 3) * 256);
        const i32x4 ia = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp);
        const i32x4 ib = *reinterpret_cast<const i32x4 *>(ids + 8 * jgrp + 4);
        const int32_t kid[8] = {ia.x, ia.y, ia.z, ia.w, ib.x, ib.y, ib.z, ib.w};
        if constexpr (WHOLE) {
#pragma unroll
            for (int i = 0; i < 32; ++i)
                copy16_nt(pool + int64_t(ids[2 * i + (lane >> 5)]) * row_bytes + 16 * (lane & 31), area + i * 1024);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    copy16_nt(pool + int64_t(kid[i]) * row_bytes + 128 * v + 16 * (lane & 7),
                              area + (8 * v + i) * 1024);
        }
        if (tail) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
                copy16_nt(pool + int64_t(ids[16 * v + (lane >> 2)]) * row_bytes + 512 + 16 * (lane & 3),
                          area + 32 * 1024);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // the id reads are done
        load_ids(k + 2);   // into the slot of ids(k - 2), read two iterations ago
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace
}  // namespace gqa

extern "C" int bw_stream_read(const void *src, size_t bytes, int64_t ctas, gqa_stream_t s) {
    if (!src || ctas < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(src) & 15u) return GQA_ERR_UNSUPPORTED;
    if (ctas > (int64_t(1) << 20) || bytes % (size_t(ctas) * 4096)) return GQA_ERR_UNSUPPORTED;
    if (bytes == 0) return GQA_OK;
    hipLaunchKernelGGL(gqa::stream_read_kernel, dim3(unsigned(ctas)), dim3(gqa::kStreamThreads), 0,
                       reinterpret_cast<hipStream_t>(s), static_cast<const uint8_t *>(src),
                       int64_t(bytes / size_t(ctas)));
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        gqa::set_error_detail(hipGetErrorString(err));
        return GQA_ERR_LAUNCH_FAILED;
    }
    return GQA_OK;
}

namespace {
int gather_rows(bool whole, const void *pool, int64_t row_bytes, const int32_t *idx, int64_t n, int64_t ctas,
                gqa_stream_t s) {
    if (!pool || !idx || n < 0 || ctas < 1) return GQA_ERR_INVALID_ARGUMENT;
    if ((row_bytes != 576 && row_bytes != 512) || (reinterpret_cast<uintptr_t>(pool) & 15u) ||
        (reinterpret_cast<uintptr_t>(idx) & 15u) || n % 64 || ctas > (int64_t(1) << 20))
        return GQA_ERR_UNSUPPORTED;
    if (n == 0) return GQA_OK;
    if (whole)
        hipLaunchKernelGGL(gqa::gather_rows_kernel<true>, dim3(unsigned(ctas)), dim3(gqa::kGatherThreads), 0,
                           reinterpret_cast<hipStream_t>(s), static_cast<const uint8_t *>(pool), row_bytes,
                           idx, n);
    else
        hipLaunchKernelGGL(gqa::gather_rows_kernel<false>, dim3(unsigned(ctas)), dim3(gqa::kGatherThreads), 0,
                           reinterpret_cast<hipStream_t>(s), static_cast<const uint8_t *>(pool), row_bytes,
                           idx, n);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) {
        gqa::set_error_detail(hipGetErrorString(err));
        return GQA_ERR_LAUNCH_FAILED;
    }
    return GQA_OK;
}
}  // namespace

extern "C" int bw_gather_rows(const void *pool, int64_t row_bytes, const int32_t *idx, int64_t n,
                              int64_t ctas, gqa_stream_t s) {
    return gather_rows(false, pool, row_bytes, idx, n, ctas, s);
}

extern "C" int bw_gather_whole_rows(const void *pool, int64_t row_bytes, const int32_t *idx, int64_t n,
                                    int64_t ctas, gqa_stream_t s) {
    return gather_rows(true, pool, row_bytes, idx, n, ctas, s);
}
