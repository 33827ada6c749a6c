// kernels.hpp -- internal interface between the C-ABI host code and the gfx950 kernels.
// Not installed; the public interface is include/gqa_splits.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gqa {

// Absorbed-MLA split kernel (fused fp8 rows: K = the whole row, V = its first DV bytes).
struct MlaSplitArgs {
    const uint16_t *q;            // bf16 [tokens, H, DQK - 64], element strides below
    int64_t q_st_tok, q_st_head;
    const uint16_t *q_pe;         // bf16 [tokens, H, 64]
    int64_t qpe_st_tok, qpe_st_head;
    const uint8_t *kv;            // fp8 rows, or bf16 rows (kv_bf16)
    int64_t kv_stride;            // bytes between rows
    const int32_t *kv_indices, *kv_indptr, *seq_lens;
    const uint8_t *kv2;           // second cache (rows of the pool's format), or null
    int64_t kv2_stride;
    const int32_t *kv2_indices, *kv2_indptr;   // request b's second-cache rows, after its pool keys
    const int32_t *glen;          // global lengths under context parallelism (cp_world > 1)
    int32_t cp_rank, cp_world;    // key j is global position j * cp_world + cp_rank
    int32_t q_len, H, np, rows_per_req, row_blocks, total_ctas;
    int32_t block_k;              // partition lengths are rounded up to a multiple of this
    // length-proportional partitions (null: np equal partitions per request): request b owns
    // slots part_start[b] .. part_start[b + 1] - 1 of part_chunk[b] keys each, and the partials
    // are then slot-major: [slot, rows_per_req, DV] and [slot, rows_per_req]
    const int32_t *part_start, *part_chunk;
    int32_t batch;
    float score_scale;            // scale * kv_scale * log2(e): scores in base-2 units
    float out_scale;              // kv_scale: the stored values are accumulated unscaled
    float *part_o;                // [rows, np, DV]
    float *part_lse2;             // [rows, np]
    uint16_t *out;                // bf16 [rows, DV] when np == 1 (direct mode)
    float *lse2_out;              // [rows] in direct mode (may be null)
};

// Grouped-query split kernel over bf16 K/V pages (head dim 128).
struct GqaSplitArgs {
    const uint16_t *q;            // bf16 [tokens, Hq, 128]
    int64_t q_st_tok, q_st_head;
    const uint16_t *k_cache, *v_cache;  // bf16 [pages, page_size, Hkv, 128]
    const int32_t *page_indices, *kv_indptr, *seq_lens;
    int32_t batch, q_len, Hq, Hkv, group, page_shift, np, total_ctas;
    int32_t block_k;              // partition lengths are rounded up to a multiple of this
    const int32_t *part_start, *part_chunk;   // as in MlaSplitArgs
    float score_scale;            // scale * log2(e)
    float *part_o, *part_lse2;
    uint16_t *out;
    float *lse2_out;
};

struct ReduceArgs {
    const float *part_o, *part_lse2;
    uint16_t *out;                // bf16 [rows, dv] (or out_f32)
    float *out_f32;               // fp32 [rows, dv] instead, when not null
    float *lse2_out;
    int64_t rows;
    int32_t np, dv;
    // element strides: partial output (row, partition) and partial lse2 (row, partition)
    int64_t o_row, o_part, l_row, l_part;
    // planned slots (null: np partitions per row): the partitions of row r of request b are
    // slots part_start[b] .. part_start[b + 1] - 1, slot-major ([slot, rows_per_req, dv]);
    // np is then only the most any request has
    const int32_t *part_start;
    int64_t rows_per_req;
};

// Device-side planner of length-proportional partitions.  Keys of request b: seq_lens[b] plus
// extra_indptr[b + 1] - extra_indptr[b] when extra_indptr is set.  Under a common length c,
// request b takes ceil(L_b / c) slots of c keys, or, beyond cap, cap slots' worth at the
// smallest multiple of block_k that fits; c is the smallest multiple of block_k whose slots
// sum to at most budget (at most one slot per request if none does).  Writes part_start
// [batch + 1] and part_chunk [batch].
struct PlanArgs {
    const int32_t *seq_lens, *extra_indptr;
    int32_t batch, budget, cap, block_k;
    int32_t *part_start, *part_chunk;
};

// Launchers: return hipSuccess or the launch error.  All enqueue on `s` only.
// Query rows one MLA split CTA covers (row_blocks = ceil(rows per request / this)).
int mla_rows_per_cta();
hipError_t launch_mla_split(const MlaSplitArgs &a, int d_qk, int d_v, bool kv_bf16, bool direct, hipStream_t s);
// (with a.kv2 set: the second-cache variant of the same kernel)
// The four-wave MLA split kernel (fp8 rows, one cache): same arguments and results as
// launch_mla_split.
hipError_t launch_mla_wide(const MlaSplitArgs &a, int d_qk, int d_v, bool direct, hipStream_t s);
// Kv heads per CTA of the GQA split when its kv-head-pair kernel runs (an even number of kv
// heads, at most 16 query rows per head group: 2, the CTA copying both heads' rows of a token as
// one run), or 0 when the one-head kernel runs (one CTA per request, partition and kv head).  The
// launch has num_kv_heads / that many CTAs per request and partition.
int gqa_heads_per_cta(int num_kv_heads, int rows_per_group);
hipError_t launch_gqa_split(const GqaSplitArgs &a, bool direct, hipStream_t s);
hipError_t launch_splitk_reduce(const ReduceArgs &a, hipStream_t s);
hipError_t launch_plan_proportional(const PlanArgs &a, hipStream_t s);
hipError_t launch_fp8_to_bf16(const uint8_t *in, int64_t n, uint16_t *out, hipStream_t s);

// Sets the text last_error_detail() returns on this thread (host code of the C ABI).
void set_error_detail(const char *msg);

}  // namespace gqa
