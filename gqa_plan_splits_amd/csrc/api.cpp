// api.cpp -- the C ABI declared in include/gqa_splits.h: argument checks, planning glue and
// kernel dispatch.  Every check runs on the host before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>

#include "../../include/gqa_splits.h"
#include "kernels.hpp"

namespace {

constexpr int kMaxPartitions = 256;
constexpr int kGqaHeadDim = 128;
constexpr int kGqaMaxRowsPerCta = 64;
constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
int ilog2(int64_t x) {
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

thread_local char g_last_error[200] = "";

}  // namespace

void gqa::set_error_detail(const char *msg) { snprintf(g_last_error, sizeof g_last_error, "%s", msg); }

namespace {

int launch_status(hipError_t err, const char *what) {
    if (err == hipSuccess) return GQA_OK;
    snprintf(g_last_error, sizeof g_last_error, "%s: %s (%d)", what, hipGetErrorString(err), int(err));
    return GQA_ERR_LAUNCH_FAILED;
}

struct Derived {
    int64_t rows;           // B * q_len * H
    int64_t rows_per_req;   // q_len * H
    int64_t cta_rows;       // CTAs per request and partition: MLA, the kernel's row blocks; GQA, kv heads
    int64_t hpg;            // heads_per_group the planner sees
    bool is_mla;
};

int check_problem(const gqa_decode_problem *p, Derived *d) {
    if (!p) return GQA_ERR_INVALID_ARGUMENT;
    if (p->batch < 1 || p->q_len < 1 || p->num_heads < 1 || p->max_num_keys < 0)
        return GQA_ERR_INVALID_ARGUMENT;
    if (!p->q || !p->kv_indices || !p->kv_indptr || !p->seq_lens) return GQA_ERR_INVALID_ARGUMENT;
    if (!(p->scale > 0.f) || !std::isfinite(p->scale)) return GQA_ERR_INVALID_ARGUMENT;
    if (p->num_heads > 128) return GQA_ERR_UNSUPPORTED;
    const int64_t rows_per_req = p->q_len * p->num_heads;
    const int64_t rows = p->batch * rows_per_req;
    if (rows_per_req > (int64_t(1) << 20) || rows > (int64_t(1) << 30)) return GQA_ERR_UNSUPPORTED;
    if (p->q_stride_tok % 8 || p->q_stride_head % 8 || !aligned16(p->q)) return GQA_ERR_UNSUPPORTED;

    if (p->kind == GQA_KIND_MLA_FUSED) {
        if (p->fp8_format != GQA_FP8_E4M3FN && p->fp8_format != GQA_FP8_E4M3FNUZ &&
            p->fp8_format != GQA_KV_BF16)
            return GQA_ERR_INVALID_ARGUMENT;
        if (!p->kv || !p->q_pe || p->num_kv_heads != 1) return GQA_ERR_INVALID_ARGUMENT;
        if (!(p->kv_scale > 0.f) || !std::isfinite(p->kv_scale)) return GQA_ERR_INVALID_ARGUMENT;
        // gfx950 converts OCP e4m3fn natively; the fnuz encoding has no kernel in this library.
        if (p->fp8_format == GQA_FP8_E4M3FNUZ) return GQA_ERR_UNSUPPORTED;
        const bool wide = p->d_qk == 576 && p->d_rope == 64 && p->d_v == 512;
        const bool sparse = p->d_qk == 512 && p->d_rope == 64 && p->d_v == 448;
        if (!wide && !sparse) return GQA_ERR_UNSUPPORTED;
        if (p->page_size != 1) return GQA_ERR_UNSUPPORTED;
        const int64_t elem = p->fp8_format == GQA_KV_BF16 ? 2 : 1;
        // (row strides below 2^32 bytes: the kernels address a row with one 32 x 32-bit product)
        if (p->kv_stride_row < p->d_qk * elem || p->kv_stride_row % 16 || p->kv_stride_row >= (int64_t(1) << 32) ||
            !aligned16(p->kv))
            return GQA_ERR_UNSUPPORTED;
        if (p->q_pe_stride_tok % 8 || p->q_pe_stride_head % 8 || !aligned16(p->q_pe))
            return GQA_ERR_UNSUPPORTED;
        // decode context parallelism: wide rows, a rank within the world, the global lengths
        if (p->cp_world > 1 || p->glen) {
            if (!p->glen || p->cp_rank < 0 || p->cp_rank >= p->cp_world) return GQA_ERR_INVALID_ARGUMENT;
            if (!wide || p->cp_world > kMaxPartitions) return GQA_ERR_UNSUPPORTED;
        } else if (p->cp_rank != 0 || p->cp_world < 0) {
            return GQA_ERR_INVALID_ARGUMENT;
        }
        // a second cache: q_len 1 without context parallelism, rows of the pool's format
        if (p->kv2 || p->kv2_indices || p->kv2_indptr) {
            if (!p->kv2 || !p->kv2_indices || !p->kv2_indptr) return GQA_ERR_INVALID_ARGUMENT;
            if (p->q_len != 1 || p->cp_world > 1 || p->glen || !sparse) return GQA_ERR_UNSUPPORTED;
            // the kernel addresses both caches with the pool's row stride
            if (p->kv2_stride_row != 0 && p->kv2_stride_row != p->kv_stride_row) return GQA_ERR_UNSUPPORTED;
            if (!aligned16(p->kv2)) return GQA_ERR_UNSUPPORTED;
        }
        d->is_mla = true;
        // the tile rule counts the CTAs the launch has: the kernel's own row blocks
        d->cta_rows = (rows_per_req + gqa::mla_rows_per_cta() - 1) / gqa::mla_rows_per_cta();
        d->hpg = rows_per_req;
    } else if (p->kind == GQA_KIND_GQA_PAGED) {
        if (!p->k_cache || !p->v_cache || p->num_kv_heads < 1) return GQA_ERR_INVALID_ARGUMENT;
        if (p->cp_world > 1 || p->glen) return GQA_ERR_UNSUPPORTED;
        if (p->kv2 || p->kv2_indices || p->kv2_indptr) return GQA_ERR_UNSUPPORTED;
        if (p->cp_rank != 0 || p->cp_world < 0) return GQA_ERR_INVALID_ARGUMENT;
        if (p->num_heads % p->num_kv_heads) return GQA_ERR_INVALID_ARGUMENT;
        if (p->d_qk != kGqaHeadDim || p->d_v != kGqaHeadDim || p->d_rope != 0)
            return GQA_ERR_UNSUPPORTED;
        if (!pow2(p->page_size) || p->page_size < 8 || p->page_size > (int64_t(1) << 20))
            return GQA_ERR_UNSUPPORTED;
        if (p->q_len * (p->num_heads / p->num_kv_heads) > kGqaMaxRowsPerCta) return GQA_ERR_UNSUPPORTED;
        if (!aligned16(p->k_cache) || !aligned16(p->v_cache)) return GQA_ERR_UNSUPPORTED;
        d->is_mla = false;
        d->cta_rows = p->num_kv_heads;
        d->hpg = p->num_kv_heads;
    } else {
        return GQA_ERR_INVALID_ARGUMENT;
    }
    d->rows = rows;
    d->rows_per_req = rows_per_req;
    return GQA_OK;
}

int resolve_plan(const gqa_decode_problem *p, const Derived &d, int64_t np_or_0, int bk_or_0,
                 int64_t sm, int64_t *np_out, int *bk_out) {
    if (np_or_0 < 0 || np_or_0 > kMaxPartitions) return GQA_ERR_UNSUPPORTED;
    if (bk_or_0 != 0 && bk_or_0 != 32 && bk_or_0 != 64) return GQA_ERR_UNSUPPORTED;
    if ((np_or_0 == 0 || bk_or_0 == 0) && sm <= 0) {
        const int rc = device_sm_count(&sm);
        if (rc != GQA_OK) return rc;
    }
    int64_t np = np_or_0;
    if (np == 0) {
        const int rc = plan_splits(p->batch, p->max_num_keys, d.hpg, sm, d.is_mla ? 1 : 0, &np);
        if (rc != GQA_OK) return rc;
    }
    int bk = bk_or_0;
    if (bk == 0) {
        bk = block_k_for(p->batch * np * d.cta_rows, sm);
        if (bk < 0) return bk;
    }
    *np_out = np;
    *bk_out = bk;
    return GQA_OK;
}

// np equal partitions per request, or with part_start set the planned length-proportional
// slots: `slots` of them in the grid, np slots per row in the partial buffers.
int launch_split(const gqa_decode_problem *p, const Derived &d, int64_t np, int bk,
                 float *part_o, float *part_lse2, void *out, float *lse2_out, hipStream_t s,
                 const int32_t *part_start = nullptr, const int32_t *part_chunk = nullptr,
                 int64_t slots = 0) {
    const bool direct = out != nullptr;
    const int64_t grid_parts = part_start ? slots : p->batch * np;
    if (d.is_mla) {
        const int64_t row_blocks = d.cta_rows;
        const int64_t total = grid_parts * row_blocks;
        if (total > (int64_t(1) << 30)) return GQA_ERR_UNSUPPORTED;
        gqa::MlaSplitArgs a;
        a.q = static_cast<const uint16_t *>(p->q);
        a.q_st_tok = p->q_stride_tok;
        a.q_st_head = p->q_stride_head;
        a.q_pe = static_cast<const uint16_t *>(p->q_pe);
        a.qpe_st_tok = p->q_pe_stride_tok;
        a.qpe_st_head = p->q_pe_stride_head;
        a.kv = static_cast<const uint8_t *>(p->kv);
        a.kv_stride = p->kv_stride_row;
        a.kv_indices = p->kv_indices;
        a.kv_indptr = p->kv_indptr;
        a.seq_lens = p->seq_lens;
        a.kv2 = static_cast<const uint8_t *>(p->kv2);
        a.kv2_stride = p->kv_stride_row;
        a.kv2_indices = p->kv2_indices;
        a.kv2_indptr = p->kv2_indptr;
        const bool cp = p->cp_world > 1 || p->glen;
        a.glen = cp ? p->glen : nullptr;
        a.cp_rank = cp ? p->cp_rank : 0;
        a.cp_world = cp ? p->cp_world : 1;
        a.q_len = int32_t(p->q_len);
        a.H = int32_t(p->num_heads);
        a.np = int32_t(np);
        a.rows_per_req = int32_t(d.rows_per_req);
        a.row_blocks = int32_t(row_blocks);
        a.total_ctas = int32_t(total);
        a.block_k = bk;
        a.part_start = part_start;
        a.part_chunk = part_chunk;
        a.batch = int32_t(p->batch);
        a.score_scale = p->scale * p->kv_scale * kLog2e;
        a.out_scale = p->kv_scale;
        a.part_o = part_o;
        a.part_lse2 = part_lse2;
        a.out = static_cast<uint16_t *>(out);
        a.lse2_out = lse2_out;
        const hipError_t err = gqa::launch_mla_split(a, int(p->d_qk), int(p->d_v),
                                                     p->fp8_format == GQA_KV_BF16, direct, s);
        return launch_status(err, "mla split");
    } else {
        // one CTA per kv head, or one per pair of kv heads
        const int hc = gqa::gqa_heads_per_cta(int(p->num_kv_heads), int(d.rows_per_req / p->num_kv_heads));
        const int64_t total = grid_parts * (hc ? p->num_kv_heads / hc : d.cta_rows);
        if (total > (int64_t(1) << 30)) return GQA_ERR_UNSUPPORTED;
        gqa::GqaSplitArgs a;
        a.q = static_cast<const uint16_t *>(p->q);
        a.q_st_tok = p->q_stride_tok;
        a.q_st_head = p->q_stride_head;
        a.k_cache = static_cast<const uint16_t *>(p->k_cache);
        a.v_cache = static_cast<const uint16_t *>(p->v_cache);
        a.page_indices = p->kv_indices;
        a.kv_indptr = p->kv_indptr;
        a.seq_lens = p->seq_lens;
        a.batch = int32_t(p->batch);
        a.q_len = int32_t(p->q_len);
        a.Hq = int32_t(p->num_heads);
        a.Hkv = int32_t(p->num_kv_heads);
        a.group = int32_t(p->num_heads / p->num_kv_heads);
        a.page_shift = ilog2(p->page_size);
        a.np = int32_t(np);
        a.total_ctas = int32_t(total);
        a.score_scale = p->scale * kLog2e;
        a.part_o = part_o;
        a.part_lse2 = part_lse2;
        a.out = static_cast<uint16_t *>(out);
        a.lse2_out = lse2_out;
        a.block_k = bk;
        a.part_start = part_start;
        a.part_chunk = part_chunk;
        const hipError_t err = gqa::launch_gqa_split(a, direct, s);
        return launch_status(err, "gqa split");
    }
}

int partial_bytes(const Derived &d, int64_t np, int64_t dv, size_t *o_bytes, size_t *l_bytes) {
    *o_bytes = align256(size_t(d.rows) * size_t(np) * size_t(dv) * sizeof(float));
    *l_bytes = align256(size_t(d.rows) * size_t(np) * sizeof(float));
    return GQA_OK;
}

}  // namespace

extern "C" int decode_plan(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0,
                           int64_t sm_count, int64_t *np_out, int *block_k_out) {
    if (!np_out || !block_k_out) return GQA_ERR_INVALID_ARGUMENT;
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    return resolve_plan(p, d, np_or_0, block_k_or_0, sm_count, np_out, block_k_out);
}

extern "C" int decode_split(const gqa_decode_problem *p, int64_t np, int block_k,
                            float *partial_o, float *partial_lse2, gqa_stream_t s) {
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    if (!partial_o || !partial_lse2) return GQA_ERR_INVALID_ARGUMENT;
    if (np < 1 || np > kMaxPartitions || (block_k != 32 && block_k != 64)) return GQA_ERR_UNSUPPORTED;
    return launch_split(p, d, np, block_k, partial_o, partial_lse2, nullptr, nullptr,
                        reinterpret_cast<hipStream_t>(s));
}

namespace {

// The merge behind splitk_reduce, splitk_reduce_f32 and merge_ranks: np inputs per row with the
// given element strides, bf16 or fp32 output.
int launch_merge(int64_t rows, int64_t np, int64_t d_v, const float *po, const float *pl,
                 void *out, bool f32_out, float *lse2_out, int64_t o_row, int64_t o_part,
                 int64_t l_row, int64_t l_part, gqa_stream_t s, const char *what) {
    if (rows < 0 || !po || !pl || !out) return GQA_ERR_INVALID_ARGUMENT;
    if (np < 1 || np > kMaxPartitions || d_v < 4 || d_v > 1024 || d_v % 4) return GQA_ERR_UNSUPPORTED;
    if (rows > (int64_t(1) << 30)) return GQA_ERR_UNSUPPORTED;
    if (!aligned16(po) || reinterpret_cast<uintptr_t>(out) % (f32_out ? 16 : 8)) return GQA_ERR_UNSUPPORTED;
    if (rows == 0) return GQA_OK;
    gqa::ReduceArgs a;
    a.part_o = po;
    a.part_lse2 = pl;
    a.out = f32_out ? nullptr : static_cast<uint16_t *>(out);
    a.out_f32 = f32_out ? static_cast<float *>(out) : nullptr;
    a.lse2_out = lse2_out;
    a.rows = rows;
    a.np = int32_t(np);
    a.dv = int32_t(d_v);
    a.o_row = o_row;
    a.o_part = o_part;
    a.l_row = l_row;
    a.l_part = l_part;
    a.part_start = nullptr;
    a.rows_per_req = 0;
    return launch_status(gqa::launch_splitk_reduce(a, reinterpret_cast<hipStream_t>(s)), what);
}

}  // namespace

extern "C" int splitk_reduce(int64_t rows, int64_t np, int64_t d_v, const float *partial_o,
                             const float *partial_lse2, void *out, float *lse2_out,
                             gqa_stream_t s) {
    // [rows, np, d_v] and [rows, np]
    return launch_merge(rows, np, d_v, partial_o, partial_lse2, out, false, lse2_out, np * d_v, d_v,
                        np, 1, s, "splitk_reduce");
}

extern "C" int splitk_reduce_f32(int64_t rows, int64_t np, int64_t d_v, const float *partial_o,
                                 const float *partial_lse2, float *out, float *lse2_out,
                                 gqa_stream_t s) {
    return launch_merge(rows, np, d_v, partial_o, partial_lse2, out, true, lse2_out, np * d_v, d_v,
                        np, 1, s, "splitk_reduce_f32");
}

extern "C" int merge_ranks(int64_t world, int64_t rows, int64_t d_v, const float *parts,
                           const float *lse2, void *out, float *lse2_out, gqa_stream_t s) {
    // [world, rows, d_v] and [world, rows]
    return launch_merge(rows, world, d_v, parts, lse2, out, false, lse2_out, d_v, rows * d_v, 1, rows,
                        s, "merge_ranks");
}

extern "C" int decode_workspace_bytes(const gqa_decode_problem *p, int64_t np, size_t *bytes) {
    if (!bytes) return GQA_ERR_INVALID_ARGUMENT;
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    if (np == 0) {
        int bk;
        rc = resolve_plan(p, d, 0, 64, 0, &np, &bk);
        if (rc != GQA_OK) return rc;
    }
    if (np < 1 || np > kMaxPartitions) return GQA_ERR_UNSUPPORTED;
    if (np == 1) {
        *bytes = 0;
        return GQA_OK;
    }
    size_t ob, lb;
    partial_bytes(d, np, p->d_v, &ob, &lb);
    *bytes = ob + lb;
    return GQA_OK;
}

extern "C" int decode(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0,
                      void *workspace, size_t ws_bytes, void *out, float *lse2_out,
                      gqa_stream_t s) {
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    if (!out) return GQA_ERR_INVALID_ARGUMENT;
    int64_t np;
    int bk;
    rc = resolve_plan(p, d, np_or_0, block_k_or_0, 0, &np, &bk);
    if (rc != GQA_OK) return rc;
    const hipStream_t st = reinterpret_cast<hipStream_t>(s);
    if (np == 1) return launch_split(p, d, 1, bk, nullptr, nullptr, out, lse2_out, st);
    size_t ob, lb;
    partial_bytes(d, np, p->d_v, &ob, &lb);
    if (!workspace) return GQA_ERR_INVALID_ARGUMENT;
    if (ws_bytes < ob + lb) return GQA_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GQA_ERR_INVALID_ARGUMENT;
    float *part_o = static_cast<float *>(workspace);
    float *part_l = reinterpret_cast<float *>(static_cast<char *>(workspace) + ob);
    rc = launch_split(p, d, np, bk, part_o, part_l, nullptr, nullptr, st);
    if (rc != GQA_OK) return rc;
    return splitk_reduce(d.rows, np, p->d_v, part_o, part_l, out, lse2_out, s);
}

extern "C" int fp8_e4m3_to_bf16(const void *in, int64_t n, void *out, gqa_stream_t s) {
    if (!in || !out || n < 0) return GQA_ERR_INVALID_ARGUMENT;
    if (!aligned16(in) || !aligned16(out)) return GQA_ERR_UNSUPPORTED;
    if (n == 0) return GQA_OK;
    return launch_status(gqa::launch_fp8_to_bf16(static_cast<const uint8_t *>(in), n,
                                                 static_cast<uint16_t *>(out),
                                                 reinterpret_cast<hipStream_t>(s)),
                         "fp8 conversion");
}

extern "C" const char *last_error_detail(void) { return g_last_error; }

extern "C" const char *status_string(int status) {
    switch (status) {
        case GQA_OK: return "ok";
        case GQA_ERR_INVALID_ARGUMENT: return "invalid argument";
        case GQA_ERR_UNSUPPORTED: return "unsupported problem for this library";
        case GQA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
        case GQA_ERR_LAUNCH_FAILED: return "kernel launch failed";
        case GQA_ERR_DEVICE: return "no usable HIP device";
        default: return "unknown status";
    }
}

namespace {

// Proportional plan: the budget of partition slots (np per request), the most one request may
// take, and the workspace layout: slot-major partials ([budget, rows_per_req, d_v] and
// [budget, rows_per_req] fp32), then part_start and part_chunk.
struct PropLayout {
    int64_t budget, cap;
    size_t o_bytes, l_bytes, start_bytes, chunk_bytes;
    size_t total() const { return o_bytes + l_bytes + start_bytes + chunk_bytes; }
};

int prop_layout(const gqa_decode_problem *p, const Derived &d, int64_t np, int64_t cap_or_0,
                PropLayout *L) {
    if (p->cp_world > 1 || p->glen) return GQA_ERR_UNSUPPORTED;
    if (np < 1 || np > kMaxPartitions || cap_or_0 < 0 || cap_or_0 > kMaxPartitions)
        return GQA_ERR_UNSUPPORTED;
    L->budget = p->batch * np;
    if (L->budget > (int64_t(1) << 30)) return GQA_ERR_UNSUPPORTED;
    L->cap = cap_or_0 ? cap_or_0 : kMaxPartitions;
    // the same bytes as np partitions per row
    partial_bytes(d, np, p->d_v, &L->o_bytes, &L->l_bytes);
    L->start_bytes = align256(size_t(p->batch + 1) * sizeof(int32_t));
    L->chunk_bytes = align256(size_t(p->batch) * sizeof(int32_t));
    return GQA_OK;
}

}  // namespace

extern "C" int plan_proportional_device(const int32_t *seq_lens, const int32_t *extra_indptr,
                                        int64_t batch, int64_t budget, int64_t cap, int block_k,
                                        int32_t *part_start, int32_t *part_chunk, gqa_stream_t s) {
    if (!seq_lens || !part_start || !part_chunk) return GQA_ERR_INVALID_ARGUMENT;
    if (batch < 1 || budget < 1 || cap < 1) return GQA_ERR_INVALID_ARGUMENT;
    if (batch > (int64_t(1) << 24) || budget > (int64_t(1) << 30) || cap > kMaxPartitions ||
        (block_k != 32 && block_k != 64))
        return GQA_ERR_UNSUPPORTED;
    gqa::PlanArgs a;
    a.seq_lens = seq_lens;
    a.extra_indptr = extra_indptr;
    a.batch = int32_t(batch);
    a.budget = int32_t(budget);
    a.cap = int32_t(cap);
    a.block_k = block_k;
    a.part_start = part_start;
    a.part_chunk = part_chunk;
    return launch_status(gqa::launch_plan_proportional(a, reinterpret_cast<hipStream_t>(s)),
                         "plan_proportional_device");
}

extern "C" int decode_proportional_workspace_bytes(const gqa_decode_problem *p, int64_t np,
                                                   int64_t cap_or_0, size_t *bytes) {
    if (!bytes) return GQA_ERR_INVALID_ARGUMENT;
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    if (np == 0) {
        int bk;
        rc = resolve_plan(p, d, 0, 64, 0, &np, &bk);
        if (rc != GQA_OK) return rc;
    }
    PropLayout L;
    rc = prop_layout(p, d, np, cap_or_0, &L);
    if (rc != GQA_OK) return rc;
    *bytes = L.total();
    return GQA_OK;
}

extern "C" int decode_proportional(const gqa_decode_problem *p, int64_t np_or_0, int64_t cap_or_0,
                                   int block_k_or_0, void *workspace, size_t ws_bytes, void *out,
                                   float *lse2_out, gqa_stream_t s) {
    Derived d;
    int rc = check_problem(p, &d);
    if (rc != GQA_OK) return rc;
    if (!out || !workspace) return GQA_ERR_INVALID_ARGUMENT;
    int64_t np;
    int bk;
    rc = resolve_plan(p, d, np_or_0, block_k_or_0, 0, &np, &bk);
    if (rc != GQA_OK) return rc;
    PropLayout L;
    rc = prop_layout(p, d, np, cap_or_0, &L);
    if (rc != GQA_OK) return rc;
    if (ws_bytes < L.total()) return GQA_ERR_WORKSPACE_TOO_SMALL;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return GQA_ERR_INVALID_ARGUMENT;
    if (reinterpret_cast<uintptr_t>(out) % 8) return GQA_ERR_UNSUPPORTED;
    char *w = static_cast<char *>(workspace);
    float *part_o = reinterpret_cast<float *>(w);
    float *part_l = reinterpret_cast<float *>(w + L.o_bytes);
    int32_t *start = reinterpret_cast<int32_t *>(w + L.o_bytes + L.l_bytes);
    int32_t *chunk = reinterpret_cast<int32_t *>(w + L.o_bytes + L.l_bytes + L.start_bytes);
    const hipStream_t st = reinterpret_cast<hipStream_t>(s);
    gqa::PlanArgs a;
    a.seq_lens = p->seq_lens;
    a.extra_indptr = p->kv2 ? p->kv2_indptr : nullptr;
    a.batch = int32_t(p->batch);
    a.budget = int32_t(L.budget);
    a.cap = int32_t(L.cap);
    a.block_k = bk;
    a.part_start = start;
    a.part_chunk = chunk;
    rc = launch_status(gqa::launch_plan_proportional(a, st), "proportional plan");
    if (rc != GQA_OK) return rc;
    // at most budget slots (budget >= batch, so the plan always fits it)
    rc = launch_split(p, d, np, bk, part_o, part_l, nullptr, nullptr, st, start, chunk, L.budget);
    if (rc != GQA_OK) return rc;
    gqa::ReduceArgs r;
    r.part_o = part_o;
    r.part_lse2 = part_l;
    r.out = static_cast<uint16_t *>(out);
    r.out_f32 = nullptr;
    r.lse2_out = lse2_out;
    r.rows = d.rows;
    r.np = int32_t(L.cap);
    r.dv = int32_t(p->d_v);
    r.o_row = r.l_row = 0;   // rows are placed through the plan
    r.o_part = d.rows_per_req * p->d_v;
    r.l_part = d.rows_per_req;
    r.part_start = start;
    r.rows_per_req = d.rows_per_req;
    return launch_status(gqa::launch_splitk_reduce(r, st), "proportional reduce");
}
