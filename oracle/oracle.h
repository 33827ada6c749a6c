/*
 * oracle.h -- plain CPU oracle for split-KV attention decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  It shares no code, header, table or constant with the GPU
 * library: every value here is recomputed from the definitions on the pages it cites.
 *
 * Every floating-point result is computed in IEEE binary64 from the stored input bits, decoded
 * exactly (bf16 and fp8 e4m3 values are all exactly representable in binary64).
 *
 * Row numbering for every attention entry point: row r = (b * q_len + t) * H + h, with b the
 * request, t the draft position within the request and h the query head.
 *
 * Return value of every int function: 0 on success, -1 on an invalid argument (null pointer,
 * non-positive size, an index out of range).  Nothing is written on error.
 */
#ifndef GQA_ORACLE_H
#define GQA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exact value of one fp8 E4M3 byte: fnuz == 0 selects the OCP e4m3fn encoding (bias 7, one
 * NaN pattern per sign, max 448), fnuz != 0 the e4m3fnuz encoding (bias 8, 0x80 is the only NaN,
 * max 240).  NaN bytes return NaN. */
double oracle_e4m3_value(uint32_t byte, int fnuz);

/* Exact value of one bfloat16 bit pattern (the top half of a binary32). */
double oracle_bf16_value(uint32_t bits);

/* Partition count of the wave-aligned planner on the Modular MAX API page
 * "hip_mha_decoding_num_partitions".  Returns the count (>= 1), or -1 when batch_size,
 * heads_per_group or sm_count is not positive or num_keys is negative. */
int64_t oracle_plan_splits(int64_t batch_size, int64_t num_keys, int64_t heads_per_group,
                           int64_t sm_count, int is_mla);

/* Tile-size rule of the AITER issue "[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the
 * CU count": 32 when the launch has more CTAs than the device has CUs, else 64.  -1 on
 * non-positive arguments. */
int oracle_block_k(int64_t ctas, int64_t sm_count);

/* (num_splits, chunks_per_block) of the sparse top-k split planner on the FlashInfer API page
 * "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits".  Candidates come in chunks of 64 (16 chunks =
 * the 1024-candidate CTA index table); the grid is counted in CTAs of 16 * head_tiles heads.
 * Returns 0 and writes both outputs, or -1 on a non-positive size or head_tiles, a negative
 * candidate count, and when max_splits is below the split count the index table forces. */
int oracle_plan_sparse_splits(int64_t num_tokens, int64_t num_heads, int64_t topk,
                              int64_t extra_topk, int64_t num_sms, int64_t max_splits,
                              int64_t head_tiles, int64_t *num_splits, int64_t *chunks_per_block);

/* Unsplit softmax attention of absorbed MLA decode over a page_size-1 fp8 pool.
 *   q_lat  [B*q_len, H, d_lat]  bf16 bits, contiguous
 *   q_pe   [B*q_len, H, d_rope] bf16 bits, contiguous (may be NULL when d_rope == 0)
 *   pool   [pool_rows, d_lat + d_rope] fp8 bytes, contiguous; key j of request b is row
 *          kv_indices[kv_indptr[b] + j]; the value part is the first d_v columns of that row;
 *          a negative entry is a skipped key (it takes a list position but no weight)
 *   seq_lens[b] keys per request; row (b, t, h) sees keys 0 .. seq_lens[b] - q_len + t
 *   rows / n_rows: the rows to compute (NULL: all B*q_len*H rows in order)
 *   o_out [n_rows, d_v], lse2_out [n_rows]: output and base-2 log-sum-exp of the scores
 * A row that sees no key gets o = 0 and lse2 = -inf. */
int oracle_mla_decode(int64_t B, int64_t q_len, int64_t H, int64_t d_lat, int64_t d_rope,
                      int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                      const uint8_t *pool, int64_t pool_rows, const int32_t *kv_indices,
                      const int32_t *kv_indptr, const int32_t *seq_lens, double scale,
                      double kv_scale, int fnuz, const int64_t *rows, int64_t n_rows,
                      double *o_out, double *lse2_out, int n_threads);

/* The same over a pool of bf16 rows ([pool_rows, d_lat + d_rope] bf16 bits), dequantized by
 * kv_scale (the bf16-cache variant). */
int oracle_mla_decode_bf16(int64_t B, int64_t q_len, int64_t H, int64_t d_lat, int64_t d_rope,
                           int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                           const uint16_t *pool, int64_t pool_rows, const int32_t *kv_indices,
                           const int32_t *kv_indptr, const int32_t *seq_lens, double scale,
                           double kv_scale, const int64_t *rows, int64_t n_rows, double *o_out,
                           double *lse2_out, int n_threads);

/* oracle_mla_decode with a second cache (sparse top-k with extra candidates, q_len = 1): query b
 * attends its seq_lens[b] main-cache keys (pool rows kv_indices[kv_indptr[b] + j]) and then every
 * second-cache key, pool2 row kv2_indices[kv2_indptr[b] + j] for j < kv2_indptr[b + 1] -
 * kv2_indptr[b] (negative entries skipped), in one softmax; pool2 has the pool's row width and
 * dequantization scale.  Returns 0, or -1 on an invalid argument. */
int oracle_mla_decode_two_caches(int64_t B, int64_t H, int64_t d_lat, int64_t d_rope,
                                 int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                                 const uint8_t *pool, int64_t pool_rows,
                                 const int32_t *kv_indices, const int32_t *kv_indptr,
                                 const int32_t *seq_lens, const uint8_t *pool2,
                                 int64_t pool2_rows, const int32_t *kv2_indices,
                                 const int32_t *kv2_indptr, double scale, double kv_scale,
                                 const int64_t *rows, int64_t n_rows, double *o_out,
                                 double *lse2_out, int n_threads);
/* The same with both caches holding bf16 rows. */
int oracle_mla_decode_two_caches_bf16(int64_t B, int64_t H, int64_t d_lat, int64_t d_rope,
                                      int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                                      const uint16_t *pool, int64_t pool_rows,
                                      const int32_t *kv_indices, const int32_t *kv_indptr,
                                      const int32_t *seq_lens, const uint16_t *pool2,
                                      int64_t pool2_rows, const int32_t *kv2_indices,
                                      const int32_t *kv2_indptr, double scale, double kv_scale,
                                      const int64_t *rows, int64_t n_rows, double *o_out,
                                      double *lse2_out, int n_threads);

/* Unsplit softmax attention of grouped-query decode over bf16 K/V pages.
 *   q        [B*q_len, Hq, D] bf16 bits
 *   k_cache, v_cache [num_pages, page_size, Hkv, D] bf16 bits
 *   token j of request b lives in page kv_page_indices[kv_indptr[b] + j / page_size],
 *   slot j % page_size; query head h reads kv head h / (Hq / Hkv). */
int oracle_gqa_decode(int64_t B, int64_t q_len, int64_t Hq, int64_t Hkv, int64_t D,
                      int64_t page_size, const uint16_t *q, const uint16_t *k_cache,
                      const uint16_t *v_cache, int64_t num_pages,
                      const int32_t *kv_page_indices, const int32_t *kv_indptr,
                      const int32_t *seq_lens, double scale, const int64_t *rows,
                      int64_t n_rows, double *o_out, double *lse2_out, int n_threads);

/* Merge of per-partition results by their base-2 log-sum-exp:
 *   lse2 = log2(sum_p 2^lse2_p),  o = sum_p 2^(lse2_p - lse2) * o_p
 * partial_o [rows, np, dv], partial_lse2 [rows, np]; a partition with lse2_p = -inf carries
 * no weight; a row whose partitions are all -inf gets o = 0, lse2 = -inf. */
int oracle_lse_merge(int64_t rows, int64_t np, int64_t dv, const double *partial_o,
                     const double *partial_lse2, double *o_out, double *lse2_out);

/* Host threads the attention entry points use when n_threads <= 0 (the process's CPU
 * affinity count). */
int oracle_default_threads(void);

#ifdef __cplusplus
}
#endif

#endif
