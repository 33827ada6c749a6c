// scratch.hip -- decode_scratch: decode() with its fp32 partials in a fixed device-side array
// instead of a caller workspace, for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation).
//
// The array below lives in the library's code object: every GPU the library runs on holds its
// own copy (kScratchBytes) from the module load until the process ends.  Host code never passes
// the array's name to a kernel (in host code that name stands for a host-side shadow, not a
// device address); it uses the device address that hipGetSymbolAddress reports, queried once per
// device with that device current and cached.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <mutex>

#include "../../include/gqa_splits.h"
#include "kernels.hpp"

namespace {

constexpr size_t kScratchBytes = GQA_SCRATCH_BYTES;   // the largest partials decode_scratch takes
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (queried once per device).
int scratch_address(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GQA_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p) {
            char msg[160];
            snprintf(msg, sizeof msg, "decode_scratch: hipGetSymbolAddress failed on device %d: %s (%d)",
                     dev, hipGetErrorString(err), int(err));
            gqa::set_error_detail(msg);
            return GQA_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return GQA_OK;
}

}  // namespace

extern "C" int decode_scratch(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0,
                              void *out, float *lse2_out, gqa_stream_t s) {
    if (!out) return GQA_ERR_INVALID_ARGUMENT;
    // the plan decode() will use, and the partials it needs (argument checks included)
    int64_t np = 0;
    int bk = 0;
    int rc = decode_plan(p, np_or_0, block_k_or_0, 0, &np, &bk);
    if (rc != GQA_OK) return rc;
    size_t need = 0;
    rc = decode_workspace_bytes(p, np, &need);
    if (rc != GQA_OK) return rc;
    if (need > kScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg, "decode_scratch: %zu bytes of partials needed, the static scratch holds %zu",
                 need, kScratchBytes);
        gqa::set_error_detail(msg);
        return GQA_ERR_WORKSPACE_TOO_SMALL;
    }
    void *ws = nullptr;
    if (need > 0) {
        rc = scratch_address(&ws);
        if (rc != GQA_OK) return rc;
    }
    return decode(p, np, bk, ws, need > 0 ? kScratchBytes : 0, out, lse2_out, s);
}
