/*
 * gqa_splits.h -- C ABI of the gfx950 split-KV ("flash-decoding") attention decode library.
 *
 * The library computes attention decode over a paged KV cache in three steps:
 *
 *   1. plan     -- a wave-aligned partition count (plan_splits) and a tile size (block_k_for);
 *   2. split    -- one partial output and one base-2 log-sum-exp per (row, partition)
 *                  (decode_split);
 *   3. reduce   -- the fp32 base-2 LSE merge of up to 256 partitions (splitk_reduce).
 *
 * decode() runs the three in order on one stream.
 *
 * Sources (pages cited by title and section):
 *   [MAX]   Modular MAX API page "hip_mha_decoding_num_partitions": the planner (regime bullets,
 *           EXCEPTION paragraph, Phase 0 sweep, AMD reducer constraint, Tunables, Args).
 *   [AITER] AITER issue "[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the CU count":
 *           the CTA-keyed tile rule ("Why it is not monotonic in num_queries") and the sparse
 *           top-k workload ("Measurements").
 *   [MM]    moonmath-amd README: absorbed MLA decode ("MLA decode" usage and constraints: fused
 *           fp8 rows that are both K and V, one per-tensor kv_scale, page_size 1 slot lists,
 *           kv_indptr / seq_lens, the end-aligned draft window, in-place outputs on the caller's
 *           stream, the base-2 LSE), paged K/V for head dim 128 (gfx950 "forward_paged":
 *           caches [pages, page_size, kv_heads, D], kv_indptr counting pages, kv_page_indices),
 *           gfx950 bf16 output rounding (RTNE), a row that sees no key is 0.
 *
 * Conventions (all entry points):
 *   - Row numbering: row r = (b * q_len + t) * H + h for request b, draft position t, query
 *     head h.  Row (b, t, h) attends keys 0 .. seq_lens[b] - q_len + t of request b [MM].
 *   - Ownership: the caller owns every buffer.  The library never calls an allocator: decode()
 *     takes its scratch space as a caller-provided workspace, and decode_scratch() uses a
 *     fixed device-side array of the library's code object.  Outputs are written in place.  The
 *     only other state is the CU count and the scratch address of each device, cached on first
 *     query.
 *   - Streams: every kernel is enqueued on the caller's stream `s` (a hipStream_t; NULL is the
 *     null stream).  No entry point synchronises the host with the device, so every call can be
 *     captured into a HIP graph.
 *   - Errors: functions return GQA_OK (0) or a negative gqa_status.  Arguments are checked on
 *     the host before anything is enqueued; nothing is enqueued on error.  GQA_ERR_LAUNCH_FAILED
 *     reports a launch error from the HIP runtime.  No C++ exception crosses this interface.
 *   - Device data is not checked (that would need a device sync).  The caller guarantees:
 *     every index is in range; seq_lens[b] <= keys addressable from kv_indptr (tokens for MLA,
 *     pages * page_size for paged GQA); inputs hold no NaN or Inf.
 */
#ifndef GQA_SPLITS_H
#define GQA_SPLITS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t *gqa_stream_t;

typedef enum gqa_status {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARGUMENT = -1,   /* null pointer, non-positive size, inconsistent sizes */
    GQA_ERR_UNSUPPORTED = -2,        /* a valid problem this library has no kernel for */
    GQA_ERR_WORKSPACE_TOO_SMALL = -3,
    GQA_ERR_LAUNCH_FAILED = -4,      /* the HIP runtime refused a launch */
    GQA_ERR_DEVICE = -5              /* no usable HIP device / device query failed */
} gqa_status;

typedef enum gqa_kind {
    /* Absorbed MLA [MM]: one fused row per token (fp8, or bf16 with GQA_KV_BF16), K = the
     * whole row, V = its first d_v elements; page_size 1.  Sparse top-k decode [AITER] is this kind with one request per query
     * whose kv_indices row holds that query's top-k slots. */
    GQA_KIND_MLA_FUSED = 0,
    /* Grouped-query / multi-head decode over bf16 K and V pages [MM, forward_paged]. */
    GQA_KIND_GQA_PAGED = 1
} gqa_kind;

/* Element format of the MLA pool (and of a second cache). */
typedef enum gqa_fp8_format {
    GQA_FP8_E4M3FN = 0,    /* OCP e4m3fn: gfx950's native fp8 */
    GQA_FP8_E4M3FNUZ = 1,  /* e4m3fnuz (the gfx942 encoding used by [MM]) */
    /* bf16 rows (2 bytes per element), the same fused rows and the same per-tensor kv_scale
     * (1 for a plain bf16 cache) [AITER, closing paragraph: the bf16-cache measurement].  The
     * value part is multiplied in fp16: stored values must lie within fp16's range (|v| < 65520);
     * below 2^-14 they are rounded to fp16's subnormal step (an error under 2^-25).  A second
     * cache then holds bf16 rows too. */
    GQA_KV_BF16 = 2
} gqa_fp8_format;

typedef struct gqa_decode_problem {
    int32_t kind;          /* gqa_kind */
    int32_t fp8_format;    /* gqa_fp8_format: the MLA pool's element format (MLA only) */

    int64_t batch;         /* B: requests, >= 1 */
    int64_t q_len;         /* queries per request, >= 1 (1: decode; > 1: draft window) */
    int64_t num_heads;     /* H: query heads, 1..128 */
    int64_t num_kv_heads;  /* GQA: kv heads (num_heads % num_kv_heads == 0); MLA: 1 */
    int64_t d_qk;          /* MLA: 576 (512 latent + 64 rope) or 512 (448 + 64); GQA: 128 */
    int64_t d_rope;        /* MLA: 64; GQA: 0 */
    int64_t d_v;           /* MLA: 512 (for d_qk 576) or 448 (for d_qk 512); GQA: 128 */
    int64_t page_size;     /* MLA: 1; GQA: a power of two >= 8 */
    int64_t max_num_keys;  /* host-known max(seq_lens): the planner's num_keys [MAX, Args] */

    /* Queries, bf16.  q: [B*q_len, H, d_qk - d_rope]; q_pe: [B*q_len, H, d_rope] (NULL when
     * d_rope == 0).  Strides are in elements; the last dimension is contiguous.  Pointers
     * 16-byte aligned, strides multiples of 8. */
    const void *q;
    int64_t q_stride_tok, q_stride_head;
    const void *q_pe;
    int64_t q_pe_stride_tok, q_pe_stride_head;

    /* MLA pool: [N, d_qk] elements of fp8_format (fp8 bytes or bf16); row stride kv_stride_row
     * bytes (a multiple of 16, >= d_qk elements and below 2^32; pointer 16-byte aligned). */
    const void *kv;
    int64_t kv_stride_row;

    /* GQA caches: bf16 [num_pages, page_size, num_kv_heads, d_qk], contiguous. */
    const void *k_cache;
    const void *v_cache;

    /* MLA: kv_indices[kv_indptr[b] + j] is the pool row of key j of request b; a negative
     *      entry is a skipped key (the top-k lists' has_invalid case [AITER, Measurements]): it
     *      keeps its list position and carries no weight.
     * GQA: kv_indices[kv_indptr[b] + j / page_size] is the page of token j of request b.
     * kv_indptr: int32 [B + 1]; seq_lens: int32 [B] keys (tokens) per request. */
    const int32_t *kv_indices;
    const int32_t *kv_indptr;
    const int32_t *seq_lens;

    float scale;           /* softmax scale applied to q . k */
    float kv_scale;        /* MLA: per-tensor dequantization scale of the pool; GQA: 1 */

    /* Decode context parallelism [MM, MLA decode] (MLA with d_qk 576 only; cp_world 0 or 1 and
     * glen NULL: off).  The keys of each request are dealt over cp_world ranks by position
     * (global position p belongs to rank p % cp_world); this call holds rank cp_rank's share:
     * seq_lens[b] counts its positions and key j of request b is global position
     * j * cp_world + cp_rank.  glen: int32 [B] device, the global lengths; draft position t
     * sees the global positions 0 .. glen[b] - q_len + t.  The ranks' outputs (each with its
     * lse2) are combined by merge_ranks. */
    const int32_t *glen;
    int32_t cp_rank;
    int32_t cp_world;

    /* A second cache [FI, Parameters: extra_topk, candidate slots per token in a second cache]
     * (sparse MLA rows, d_qk 512, with q_len 1 and no context parallelism; kv2 NULL: off).
     * kv2: rows of the pool's format [N2, d_qk] at the pool's row stride (kv2_stride_row 0
     * or equal to kv_stride_row; pointer 16-byte aligned), dequantized with kv_scale.  Request b
     * attends its seq_lens[b] pool keys and then the second-cache rows
     * kv2_indices[kv2_indptr[b] .. kv2_indptr[b + 1]) (negative: skipped), all in one softmax;
     * partitions cut the concatenated list.  kv2_indptr: int32 [B + 1].  max_num_keys must cover
     * seq_lens[b] plus the request's second-cache count.  Errors: kv2 without both index lists
     * (or the reverse) GQA_ERR_INVALID_ARGUMENT; with the GQA kind, wide rows, q_len > 1,
     * context parallelism or another row stride GQA_ERR_UNSUPPORTED. */
    const void *kv2;
    int64_t kv2_stride_row;
    const int32_t *kv2_indices;
    const int32_t *kv2_indptr;
} gqa_decode_problem;

/* ---------------------------------------------------------------------------------------- */
/* Planning [MAX], [AITER]                                                                  */
/* ---------------------------------------------------------------------------------------- */

/* Partition count of the wave-aligned planner [MAX]:
 *   batch_size      requests in the batch (>= 1)
 *   num_keys        keys to scan (>= 0)
 *   heads_per_group not a group size: the kv-head count for MHA-style callers, the number of
 *                   query rows packed per request for MLA callers (>= 1)
 *   sm_count        CUs used to size the waves; <= 0 queries the current HIP device (cached)
 *   is_mla          non-zero for the MLA caller
 * Writes the count (1..256) to *np_out.  Pure host integer arithmetic when sm_count > 0.
 * Errors: INVALID_ARGUMENT (np_out NULL, batch_size/heads_per_group < 1, num_keys < 0),
 * DEVICE (sm_count <= 0 and no device). */
int plan_splits(int64_t batch_size, int64_t num_keys, int64_t heads_per_group, int64_t sm_count,
                int is_mla, int64_t *np_out);

/* Tile size in keys [AITER]: 32 when the launch has more CTAs than the device has CUs,
 * else 64.  Returns 32 or 64, or GQA_ERR_INVALID_ARGUMENT when ctas < 1 or sm_count < 1. */
int block_k_for(int64_t ctas, int64_t sm_count);

/* Split plan of the sparse top-k planner on the FlashInfer API page
 * "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits" (its measured split rules and GB10 paragraph),
 * for one decode call of sparse MLA:
 *   num_tokens   query tokens in the call (>= 1)
 *   num_heads    query heads per token (>= 1)
 *   topk         candidate slots per token in the main cache (>= 0)
 *   extra_topk   candidate slots per token in a second cache (>= 0; 0 without one)
 *   num_sms      CUs the grid is sized for; <= 0 queries the current HIP device (cached)
 *   max_splits   upper bound on the split count (>= 1)
 *   head_tiles   the grid is counted in CTAs of 16 * head_tiles heads (>= 1; this library's
 *                MLA kernel runs 64 query rows per CTA, head_tiles = 4)
 * Candidates are chunked by 64, each cache on its own.  Writes the split count to *num_splits_out
 * and ceil(chunks / splits) to *chunks_per_block_out (at most 16: the page's CTA index table).
 * Pure host integer arithmetic when num_sms > 0.  Errors: INVALID_ARGUMENT (a NULL output, a
 * size below its bound, or max_splits below the ceil(chunks / 16) splits the index table forces),
 * DEVICE (num_sms <= 0 and no device). */
int plan_sparse_splits(int64_t num_tokens, int64_t num_heads, int64_t topk, int64_t extra_topk,
                       int64_t num_sms, int64_t max_splits, int64_t head_tiles,
                       int64_t *num_splits_out, int64_t *chunks_per_block_out);

/* The wave-aligned planner's choice for paged GQA, raised where this library's GQA split kernel
 * measured better on MI355X: max(plan_splits(batch_size, max_num_keys, num_kv_heads, sm_count,
 * 0), the smallest power of two np with batch_size * num_kv_heads * np >= 4 * sm_count), the
 * latter held to at least 256 keys per partition (the largest power of two <= max_num_keys / 256,
 * at least 1) and to 256.  The kernel's CTAs are one wave and several run per CU, so the pages'
 * count of one CTA per CU under-splits batches with few kv-head CTAs.  sm_count <= 0 queries the
 * current device.  Not a rule of the pages: a measured tuning, checked by the benchmark's
 * planner-branch sweep.  Errors: INVALID_ARGUMENT (NULL output, a size below its bound), DEVICE,
 * and those of plan_splits. */
int plan_gqa_splits_measured(int64_t batch_size, int64_t max_num_keys, int64_t num_kv_heads,
                             int64_t sm_count, int64_t *np_out);

/* The partition count this library's MLA split kernel measured best on MI355X (a tuning for this
 * kernel, not a rule of the pages; plan_splits stays [MAX]'s rule): the largest power of two np
 * <= 256 with batch_size * ceil(rows_per_request / 64) * np <= sm_count -- one wave of the
 * kernel's 64-row CTAs, of which one runs per CU and hides its own read latency -- and at least
 * 256 keys (four 64-key tiles) per partition; 1 when neither allows 2.  rows_per_request is
 * q_len * H.  Where [MAX]'s EXCEPTION paragraph (MLA with <= 16 heads) asks for two waves,
 * this keeps one: a second wave of this kernel's CTAs only adds their prologues and epilogues.
 * sm_count <= 0 queries the current device.  Checked by the benchmark's planner-branch sweep.
 * Errors: INVALID_ARGUMENT (NULL output, a size below its bound), DEVICE. */
int plan_mla_splits_measured(int64_t batch_size, int64_t max_num_keys, int64_t rows_per_request,
                             int64_t sm_count, int64_t *np_out);

/* The sparse planner's decision with thresholds measured on MI355X for this library's MLA
 * kernel rather than the page's (which were measured for a Blackwell kernel): the largest power
 * of two (<= max_splits) that keeps num_tokens * ceil(num_heads / rows_per_cta) * splits within
 * sm_count CTAs and leaves every CTA at least two 64-candidate chunks (one when a single CTA runs
 * unsplit); 1 for two chunks or fewer.  No split is forced by the chunk count.  rows_per_cta is
 * the query rows one CTA runs (64 for this library's MLA kernel); sm_count <= 0 queries the
 * current device.  Not a rule of the pages: a measured tuning, checked by the benchmark's sparse
 * sweep.  Errors: INVALID_ARGUMENT (NULL output, a size below its bound), DEVICE. */
int plan_sparse_splits_measured(int64_t num_tokens, int64_t num_heads, int64_t topk,
                                int64_t extra_topk, int64_t sm_count, int64_t max_splits,
                                int64_t rows_per_cta, int64_t *num_splits_out);

/* CU count of the current HIP device, cached per device after the first query. */
int device_sm_count(int64_t *sm_out);

/* What decode() would launch: the partition count (np_or_0, or the planner's choice when 0)
 * and the tile size (block_k_or_0, or the tile rule's choice when 0), for the device with
 * sm_count CUs (<= 0: the current device).  The planner sees heads_per_group = q_len * H for
 * MLA (the query rows packed per request) and num_kv_heads for GQA; the tile rule sees the
 * CTA count of the split launch, B * np * ceil(q_len * H / 64) for MLA (the kernel's CTAs run 64
 * query rows) and B * np * num_kv_heads for GQA.  The split kernels' key tiles are fixed (MLA:
 * 64 fp8 or 32 bf16 keys; GQA: 16 tokens), so block_k sets the partitions' granularity: partition
 * lengths are rounded up to it. */
int decode_plan(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0, int64_t sm_count,
                int64_t *np_out, int *block_k_out);

/* ---------------------------------------------------------------------------------------- */
/* Split, reduce, decode                                                                    */
/* ---------------------------------------------------------------------------------------- */

/* Split kernel [MM, MLA decode: the op "splits a batch's KV by request length" and returns a
 * base-2 LSE; gfx950 forward_paged for the paged GQA kind] [MAX, Args: np partitions per
 * request]: request b's keys are cut into np contiguous partitions of
 * ceil(seq_lens[b] / np) keys rounded up to block_k (trailing partitions may be empty).  For
 * every row r and partition i it writes
 *   partial_o   [rows, np, d_v] fp32: softmax-weighted mean of the partition's values,
 *   partial_lse2[rows, np]      fp32: log2 of the sum of e^score over the partition's keys,
 * with (0, -inf) for a partition the row sees no key of.  np in 1..256, block_k 32 or 64.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (shapes outside the table at the top of the problem
 * struct, fnuz fp8, q_len * group above 64 for GQA), LAUNCH_FAILED. */
int decode_split(const gqa_decode_problem *p, int64_t np, int block_k, float *partial_o,
                 float *partial_lse2, gqa_stream_t s);

/* Reducer: for every row, lse2 = log2(sum_i 2^lse2_i) and o = sum_i 2^(lse2_i - lse2) * o_i,
 * summed in fp32 in a fixed order (deterministic); partitions with lse2_i = -inf carry no
 * weight (their partial_o is not used) and a row with none gets o = 0, lse2 = -inf [MAX, AMD
 * reducer constraint].
 *   partial_o [rows, np, d_v] fp32, partial_lse2 [rows, np] fp32 (inputs)
 *   out       [rows, d_v] bf16, rounded to nearest even (output)
 *   lse2_out  [rows] fp32 (output; may be NULL)
 * np in 1..256, d_v a multiple of 4 up to 1024; partial_o 16-byte and out 8-byte aligned
 * (UNSUPPORTED otherwise). */
int splitk_reduce(int64_t rows, int64_t np, int64_t d_v, const float *partial_o,
                  const float *partial_lse2, void *out, float *lse2_out, gqa_stream_t s);

/* The same reducer with an fp32 output [rows, d_v], 16-byte aligned (for a caller that merges
 * further: a decode-context-parallel rank hands merge_ranks its fp32 output).  Arguments and
 * errors as splitk_reduce. */
int splitk_reduce_f32(int64_t rows, int64_t np, int64_t d_v, const float *partial_o,
                      const float *partial_lse2, float *out, float *lse2_out, gqa_stream_t s);

/* Merge of the outputs of cp_world decode-context-parallel ranks [MM, MLA decode]: the same
 * base-2 LSE merge as splitk_reduce, over the ranks' outputs (decode_split then
 * splitk_reduce_f32 on each rank) stacked rank-major.
 *   parts [world, rows, d_v] fp32, lse2 [world, rows] fp32 (inputs; a rank that saw no key of a
 *   row has lse2 = -inf there and its output is not used)
 *   out   [rows, d_v] bf16 RNE (output), lse2_out [rows] fp32 (output; may be NULL)
 * world in 1..256, d_v a multiple of 4 up to 1024; parts 16-byte and out 8-byte aligned.
 * Errors: INVALID_ARGUMENT, UNSUPPORTED, LAUNCH_FAILED. */
int merge_ranks(int64_t world, int64_t rows, int64_t d_v, const float *parts, const float *lse2,
                void *out, float *lse2_out, gqa_stream_t s);

/* Workspace decode() needs for np partitions (np = 0: the planner's choice on the current
 * device): the fp32 partials, 256-byte aligned; 0 when np == 1 (the split kernel then writes
 * the final output itself).  The partials are fp32 as the reducer's inputs [MAX, AMD reducer
 * constraint] and [MM, Numerics: "the fp32 partial merge"].  Errors: those of decode_split's
 * checks, INVALID_ARGUMENT for a NULL bytes. */
int decode_workspace_bytes(const gqa_decode_problem *p, int64_t np, size_t *bytes);

/* Whole decode [MM, MLA decode usage: one call with outputs written in place on the caller's
 * stream; Numerics: deterministic, the split a function of the inputs]: plan (np_or_0 == 0 /
 * block_k_or_0 == 0 use the planner [MAX] / tile rule [AITER] on the current device), split,
 * and reduce.
 *   out      [B*q_len, H, d_v] bf16, contiguous (output)
 *   lse2_out [B*q_len, H] fp32 (output; may be NULL)
 * Errors: as decode_split, plus WORKSPACE_TOO_SMALL when ws_bytes is below
 * decode_workspace_bytes. */
int decode(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0, void *workspace,
           size_t ws_bytes, void *out, float *lse2_out, gqa_stream_t s);

/* Device-side plan of length-proportional partitions [MM, "VarlenPlan": a plan made on the GPU
 * from device-side lengths, so a captured decode replays with new lengths; the rule is this
 * library's reading].  Request b has L_b = seq_lens[b] keys, plus extra_indptr[b + 1] -
 * extra_indptr[b] when extra_indptr is not NULL (a second cache).  Under a common length c,
 * request b takes n_b = ceil(L_b / c) partitions of c keys, or, when that exceeds cap,
 * chunk_b = the smallest multiple of block_k with ceil(L_b / chunk_b) <= cap and as many
 * partitions of chunk_b keys as that needs.  c is the smallest multiple of block_k for which
 * the sum of n_b is at most budget; if none is (budget below the number of non-empty requests),
 * c is the longest L_b rounded up to block_k.  Partition j of request b covers its keys
 * [j * chunk_b, (j + 1) * chunk_b).  A negative L_b counts as 0, and one above 2^31 - 64 as
 * 2^31 - 64 (so that every chunk_b fits an int32).
 *   seq_lens [batch], extra_indptr [batch + 1] or NULL: int32 device (inputs)
 *   part_start [batch + 1] int32 device (output): exclusive prefix sum of n_b
 *   part_chunk [batch] int32 device (output): chunk_b
 * batch 1..2^24, budget 1..2^30, cap 1..256, block_k 32 or 64.  Enqueued on s, no host sync.
 * Errors: INVALID_ARGUMENT (NULL pointer, batch, budget or cap below 1), UNSUPPORTED (out of
 * range), LAUNCH_FAILED. */
int plan_proportional_device(const int32_t *seq_lens, const int32_t *extra_indptr, int64_t batch,
                             int64_t budget, int64_t cap, int block_k, int32_t *part_start,
                             int32_t *part_chunk, gqa_stream_t s);

/* Workspace decode_proportional() needs: the partials of batch * np slots, slot-major
 * ([slot, q_len * H, d_v] and [slot, q_len * H] fp32: as many bytes as decode's np partitions
 * per row), then the plan's two tables, each part 256-byte aligned.  np = 0: the planner's
 * choice on the current device; cap_or_0 (0 or 1..256) does not change the size. */
int decode_proportional_workspace_bytes(const gqa_decode_problem *p, int64_t np, int64_t cap_or_0,
                                        size_t *bytes);

/* Whole decode with length-proportional partitions planned on the device: the budget is
 * batch * np slots, the grid of the equal split (np_or_0 = 0: the planner's np), split by
 * plan_proportional_device over the problem's lengths (and second-cache counts) with at most
 * cap_or_0 (0: 256) slots per request; then the split kernel over the planned slots and the
 * reducer over each row's slots, both placed through the plan's tables.  No host sync: a
 * captured call re-plans on every replay.  Output as decode (out 8-byte aligned).  Without
 * context parallelism (else UNSUPPORTED).  Errors: as decode, WORKSPACE_TOO_SMALL below
 * decode_proportional_workspace_bytes. */
int decode_proportional(const gqa_decode_problem *p, int64_t np_or_0, int64_t cap_or_0,
                        int block_k_or_0, void *workspace, size_t ws_bytes, void *out,
                        float *lse2_out, gqa_stream_t s);

/* Bytes of the device-side scratch array decode_scratch() keeps its partials in (64 MiB per GPU). */
#define GQA_SCRATCH_BYTES ((size_t)64 << 20)

/* Allocation-free decode, for callers that cannot allocate device memory or pass a workspace
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the same
 * plan, split and reduce as decode(), with the fp32 partials in a device-side array of
 * GQA_SCRATCH_BYTES that the library's code object holds on every GPU it runs on until the
 * process ends.  Calls nothing that allocates.  The first call on a device queries that device's
 * address of the array (hipGetSymbolAddress) and caches it.
 *   out      [B*q_len, H, d_v] bf16, contiguous (output)
 *   lse2_out [B*q_len, H] fp32 (output; may be NULL)
 * The array is shared by every call on a GPU and holds the last call's partials: calls that
 * overlap on one GPU (other streams, other threads) race and must be serialized by the caller.
 * Nothing in it needs clearing (every partial a call reads, that call wrote).
 * Errors: as decode, and WORKSPACE_TOO_SMALL when the partials of the plan exceed
 * GQA_SCRATCH_BYTES (np == 1 needs none); DEVICE when the array's address cannot be queried.
 * last_error_detail() then says how many bytes were needed. */
int decode_scratch(const gqa_decode_problem *p, int64_t np_or_0, int block_k_or_0, void *out,
                   float *lse2_out, gqa_stream_t s);

/* Utility: decode n OCP e4m3fn bytes to bf16 with the same conversion the MLA split kernel
 * applies to the pool (exact; unit scale).  in, out 16-byte aligned device buffers; out holds
 * n bf16 values.  Lets callers and tests check the device's fp8 decoding byte by byte. */
int fp8_e4m3_to_bf16(const void *in, int64_t n, void *out, gqa_stream_t s);

/* ---------------------------------------------------------------------------------------- */
/* Measurement: data-movement ceilings of this GPU (for the benchmark's roofline)            */
/* ---------------------------------------------------------------------------------------- */

/* Reads `bytes` contiguous bytes of src into LDS with the copy instruction the split kernels use
 * (global_load_lds_dwordx4, non-temporal), discarding them: the streaming-read ceiling.  ctas
 * workgroups of 4 waves each read bytes / ctas contiguous bytes.  src 16-byte aligned device
 * memory; bytes a multiple of ctas * 4096.  Enqueued on s.  Errors: INVALID_ARGUMENT (NULL src,
 * ctas < 1), UNSUPPORTED (alignment, sizes), LAUNCH_FAILED. */
int bw_stream_read(const void *src, size_t bytes, int64_t ctas, gqa_stream_t s);

/* Gathers the n rows pool[idx[i] * row_bytes ..] (row_bytes 576 or 512) into LDS with the MLA split
 * kernel's copy pattern and instruction (per 64 rows: four lines of 128 bytes, 8 rows per copy,
 * and for 576-byte rows the 64-byte rope tails, 16 rows per copy), discarding them: the ceiling of
 * that kernel's gather [MM, MLA decode: page_size 1 slot lists].  ctas workgroups of 4 waves take
 * 64-row groups in turn.  pool and idx 16-byte aligned device memory; every idx[i] a pool row
 * (not checked); n a multiple of 64.  Enqueued on s.  Errors: INVALID_ARGUMENT, UNSUPPORTED,
 * LAUNCH_FAILED. */
int bw_gather_rows(const void *pool, int64_t row_bytes, const int32_t *idx, int64_t n, int64_t ctas,
                   gqa_stream_t s);

/* As bw_gather_rows, with whole-row requests: each copy instruction moves the first 512 bytes of
 * two rows (32 lanes per row), the rope tails of 576-byte rows as there.  The same rows, bytes,
 * arguments and errors; the gather ceiling of a copy pattern that keeps each row's bytes in one
 * request [MM, MLA decode: page_size 1 slot lists]. */
int bw_gather_whole_rows(const void *pool, int64_t row_bytes, const int32_t *idx, int64_t n,
                         int64_t ctas, gqa_stream_t s);

/* Static description of a status code (the error classes of the constraints lists [MM, MLA
 * decode and gfx950 constraints]: shapes outside them are UNSUPPORTED); never NULL, "unknown
 * status" for a value outside gqa_status. */
const char *status_string(int status);

/* Text behind the calling thread's most recent GQA_ERR_LAUNCH_FAILED (the HIP error) or
 * decode_scratch failure ("" if none); valid until the thread's next failing call. */
const char *last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_SPLITS_H */
