// decode_abi.cpp -- drives the C ABI of libgqa_splits.so from C++, with no Python in the process:
// device buffers from hipMalloc, seeded inputs drawn here, decode() on a stream of its own, and
// the fp64 oracle (liboracle.so, test infrastructure) over the same bytes.  Cases: absorbed MLA
// over an fp8 pool and over a bf16 pool (ragged requests, a draft window of 2, a request with no
// keys), each at the planner's np and at np = 3, and paged GQA.  Exit status 0 when every output
// meets the project bars (max|dO| <= 1e-2, max|dO| / max|O| <= 1e-2, |d lse2| <= 1e-4 max(1, |lse2|),
// rows that see no key exactly 0 and -inf).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gqa_splits.h"
#include "oracle.h"

namespace {

int g_failures = 0;

#define HIP_OK(x)                                                                            \
    do {                                                                                     \
        hipError_t e_ = (x);                                                                 \
        if (e_ != hipSuccess) {                                                              \
            std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);       \
            std::exit(2);                                                                    \
        }                                                                                    \
    } while (0)

// splitmix64: a counter-based generator (each draw a function of the seed and the counter)
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9E3779B97F4A7C15ull);
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        return z ^ (z >> 31);
    }
    double uniform() { return (next() >> 11) * (1.0 / 9007199254740992.0); }   // [0, 1)
};

// bf16 bits of a float, round to nearest even (finite inputs)
uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return uint16_t(u >> 16);
}
float from_bf16(uint16_t b) {
    uint32_t u = uint32_t(b) << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

template <typename T>
T *to_device(const std::vector<T> &h) {
    T *d = nullptr;
    HIP_OK(hipMalloc(&d, std::max<size_t>(h.size(), 1) * sizeof(T)));
    if (!h.empty()) HIP_OK(hipMemcpy(d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
    return d;
}

bool check_status(int rc, const char *what) {
    if (rc == GQA_OK) return true;
    std::printf("%s: %s (%s)\n", what, status_string(rc), last_error_detail());
    ++g_failures;
    return false;
}

// Runs decode() on the problem and compares with the oracle's (o, lse2).
void run_and_compare(const char *what, const gqa_decode_problem &p, int64_t np, int64_t rows,
                     int64_t d_v, const std::vector<double> &ref_o, const std::vector<double> &ref_l,
                     hipStream_t s) {
    size_t ws_bytes = 0;
    if (!check_status(decode_workspace_bytes(&p, np, &ws_bytes), what)) return;
    void *ws = nullptr, *out = nullptr;
    float *lse = nullptr;
    HIP_OK(hipMalloc(&ws, std::max<size_t>(ws_bytes, 256)));
    HIP_OK(hipMalloc(&out, size_t(rows) * d_v * 2));
    HIP_OK(hipMalloc(&lse, size_t(rows) * 4));
    if (check_status(decode(&p, np, 0, ws, ws_bytes, out, lse, reinterpret_cast<gqa_stream_t>(s)), what)) {
        HIP_OK(hipStreamSynchronize(s));
        std::vector<uint16_t> o(size_t(rows) * d_v);
        std::vector<float> l(rows);
        HIP_OK(hipMemcpy(o.data(), out, o.size() * 2, hipMemcpyDeviceToHost));
        HIP_OK(hipMemcpy(l.data(), lse, l.size() * 4, hipMemcpyDeviceToHost));
        double max_abs = 0, max_ref = 0, max_lse = 0;
        bool empty_ok = true;
        for (int64_t r = 0; r < rows; ++r) {
            const bool empty = std::isinf(ref_l[r]);
            if (empty != std::isinf(l[r])) empty_ok = false;
            for (int64_t c = 0; c < d_v; ++c) {
                const double v = from_bf16(o[size_t(r) * d_v + c]), w = ref_o[size_t(r) * d_v + c];
                if (empty && v != 0.0) empty_ok = false;
                max_abs = std::max(max_abs, std::fabs(v - w));
                max_ref = std::max(max_ref, std::fabs(w));
            }
            if (!empty)
                max_lse = std::max(max_lse, std::fabs(l[r] - ref_l[r]) / std::max(1.0, std::fabs(ref_l[r])));
        }
        const bool ok = empty_ok && max_abs <= 1e-2 && max_abs <= 1e-2 * max_ref && max_lse <= 1e-4;
        std::printf("%-32s np=%-3lld max|dO| %.3g rel %.3g lse2 %.3g empty-rows %s: %s\n", what,
                    (long long)np, max_abs, max_ref > 0 ? max_abs / max_ref : 0.0, max_lse,
                    empty_ok ? "ok" : "WRONG", ok ? "ok" : "FAIL");
        if (!ok) ++g_failures;
    }
    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(lse));
}

void mla_case(bool bf16_pool, hipStream_t s) {
    const int64_t B = 3, q_len = 2, H = 16, d_lat = 512, d_rope = 64, d_qk = 576, d_v = 512;
    const std::vector<int32_t> lens = {1000, 37, 0};
    const int64_t pool_rows = 1100, rows = B * q_len * H;
    Rng rng{bf16_pool ? 77u : 76u};
    std::vector<uint16_t> q_lat(size_t(B * q_len * H * d_lat)), q_pe(size_t(B * q_len * H * d_rope));
    for (auto &x : q_lat) x = to_bf16(float(2.0 * rng.uniform() - 1.0));
    for (auto &x : q_pe) x = to_bf16(float(2.0 * rng.uniform() - 1.0));
    std::vector<uint8_t> pool8;
    std::vector<uint16_t> pool16;
    if (bf16_pool) {
        pool16.resize(size_t(pool_rows * d_qk));
        for (auto &x : pool16) x = to_bf16(float(4.0 * rng.uniform() - 2.0));
    } else {
        pool8.resize(size_t(pool_rows * d_qk));
        // e4m3fn codes of magnitude up to 60 (0x67), both signs: values up to 1.9 after kv_scale,
        // so that the bf16 output's own rounding stays below the 1e-2 bar
        for (auto &x : pool8) {
            const uint64_t r = rng.next();
            x = uint8_t((r % 0x68) | ((r >> 32) & 1u) << 7);
        }
    }
    std::vector<int32_t> indptr = {0}, idx;
    for (int32_t L : lens) {
        for (int32_t j = 0; j < L; ++j) idx.push_back(int32_t(rng.next() % pool_rows));
        indptr.push_back(int32_t(idx.size()));
    }
    const double scale = 1.0 / std::sqrt(double(d_qk)), kv_scale = bf16_pool ? 1.0 : 1.0 / 32.0;
    std::vector<double> ref_o(size_t(rows * d_v)), ref_l(rows);
    const int rc = bf16_pool
        ? oracle_mla_decode_bf16(B, q_len, H, d_lat, d_rope, d_v, q_lat.data(), q_pe.data(), pool16.data(),
                                 pool_rows, idx.data(), indptr.data(), lens.data(), scale, kv_scale, nullptr,
                                 rows, ref_o.data(), ref_l.data(), 0)
        : oracle_mla_decode(B, q_len, H, d_lat, d_rope, d_v, q_lat.data(), q_pe.data(), pool8.data(),
                            pool_rows, idx.data(), indptr.data(), lens.data(), scale, kv_scale, 0, nullptr,
                            rows, ref_o.data(), ref_l.data(), 0);
    if (rc != 0) {
        std::printf("oracle rejected the MLA case\n");
        ++g_failures;
        return;
    }
    gqa_decode_problem p;
    std::memset(&p, 0, sizeof p);
    p.kind = GQA_KIND_MLA_FUSED;
    p.fp8_format = bf16_pool ? GQA_KV_BF16 : GQA_FP8_E4M3FN;
    p.batch = B;
    p.q_len = q_len;
    p.num_heads = H;
    p.num_kv_heads = 1;
    p.d_qk = d_qk;
    p.d_rope = d_rope;
    p.d_v = d_v;
    p.page_size = 1;
    p.max_num_keys = 1000;
    p.q = to_device(q_lat);
    p.q_stride_tok = H * d_lat;
    p.q_stride_head = d_lat;
    p.q_pe = to_device(q_pe);
    p.q_pe_stride_tok = H * d_rope;
    p.q_pe_stride_head = d_rope;
    p.kv = bf16_pool ? static_cast<const void *>(to_device(pool16)) : static_cast<const void *>(to_device(pool8));
    p.kv_stride_row = d_qk * (bf16_pool ? 2 : 1);
    p.kv_indices = to_device(idx);
    p.kv_indptr = to_device(indptr);
    p.seq_lens = to_device(lens);
    p.scale = float(scale);
    p.kv_scale = float(kv_scale);
    const char *what = bf16_pool ? "MLA, bf16 pool" : "MLA, fp8 pool";
    run_and_compare(what, p, 0, rows, d_v, ref_o, ref_l, s);
    run_and_compare(what, p, 3, rows, d_v, ref_o, ref_l, s);
    HIP_OK(hipFree(const_cast<void *>(p.q)));
    HIP_OK(hipFree(const_cast<void *>(p.q_pe)));
    HIP_OK(hipFree(const_cast<void *>(p.kv)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.kv_indices)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.kv_indptr)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.seq_lens)));
}

// Hq / Hkv x q_len query rows per kv head: 8 (the kv-head-pair kernel), 12 over 3 kv heads (one
// 16-row wave per kv head), 24 (two 16-row waves) and 48 (two 32-row waves).
void gqa_case(hipStream_t s, int64_t Hq, int64_t Hkv, int64_t q_len) {
    const int64_t B = 3, D = 128, page = 16, num_pages = 80;
    const std::vector<int32_t> lens = {700, 33, 1};
    const int64_t rows = B * q_len * Hq;
    Rng rng{78u};
    std::vector<uint16_t> q(size_t(rows * D)), kc(size_t(num_pages * page * Hkv * D)), vc(kc.size());
    for (auto &x : q) x = to_bf16(float(2.0 * rng.uniform() - 1.0));
    for (auto &x : kc) x = to_bf16(float(2.0 * rng.uniform() - 1.0));
    for (auto &x : vc) x = to_bf16(float(2.0 * rng.uniform() - 1.0));
    std::vector<int32_t> indptr = {0}, pages;
    int32_t next_page = 0;
    for (int32_t L : lens) {
        for (int32_t j = 0; j < (L + page - 1) / page; ++j) pages.push_back((next_page++ * 7) % int32_t(num_pages));
        indptr.push_back(int32_t(pages.size()));
    }
    const double scale = 1.0 / std::sqrt(double(D));
    std::vector<double> ref_o(size_t(rows * D)), ref_l(rows);
    if (oracle_gqa_decode(B, q_len, Hq, Hkv, D, page, q.data(), kc.data(), vc.data(), num_pages, pages.data(),
                          indptr.data(), lens.data(), scale, nullptr, rows, ref_o.data(), ref_l.data(), 0) != 0) {
        std::printf("oracle rejected the GQA case\n");
        ++g_failures;
        return;
    }
    gqa_decode_problem p;
    std::memset(&p, 0, sizeof p);
    p.kind = GQA_KIND_GQA_PAGED;
    p.batch = B;
    p.q_len = q_len;
    p.num_heads = Hq;
    p.num_kv_heads = Hkv;
    p.d_qk = D;
    p.d_v = D;
    p.page_size = page;
    p.max_num_keys = 700;
    p.q = to_device(q);
    p.q_stride_tok = Hq * D;
    p.q_stride_head = D;
    p.k_cache = to_device(kc);
    p.v_cache = to_device(vc);
    p.kv_indices = to_device(pages);
    p.kv_indptr = to_device(indptr);
    p.seq_lens = to_device(lens);
    p.scale = float(scale);
    p.kv_scale = 1.0f;
    char what[96];
    std::snprintf(what, sizeof what, "GQA, bf16 pages, %lld heads over %lld, q_len %lld", (long long)Hq,
                  (long long)Hkv, (long long)q_len);
    run_and_compare(what, p, 0, rows, D, ref_o, ref_l, s);
    run_and_compare(what, p, 3, rows, D, ref_o, ref_l, s);
    HIP_OK(hipFree(const_cast<void *>(p.q)));
    HIP_OK(hipFree(const_cast<void *>(p.k_cache)));
    HIP_OK(hipFree(const_cast<void *>(p.v_cache)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.kv_indices)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.kv_indptr)));
    HIP_OK(hipFree(const_cast<int32_t *>(p.seq_lens)));
}

}  // namespace

int main() {
    int64_t sm = 0;
    if (device_sm_count(&sm) != GQA_OK) {
        std::printf("no HIP device\n");
        return 2;
    }
    std::printf("device with %lld CUs\n", (long long)sm);
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    mla_case(false, s);
    mla_case(true, s);
    gqa_case(s, 16, 2, 1);
    gqa_case(s, 12, 3, 3);
    gqa_case(s, 24, 1, 1);
    gqa_case(s, 16, 1, 3);
    HIP_OK(hipStreamDestroy(s));
    std::printf("%s (%d failures)\n", g_failures ? "FAILED" : "all cases pass", g_failures);
    return g_failures ? 1 : 0;
}
