/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for split-KV attention decode.
 *
 * TEST INFRASTRUCTURE ONLY (tests, the smoke check and the benchmark's CPU-baseline leg).
 * It shares nothing with the GPU library.  Sources followed:
 *
 *  - Planner: Modular MAX API page "hip_mha_decoding_num_partitions" -- the MHA-style and
 *    MLA-style regime bullets, the EXCEPTION paragraph, the "Phase 0 sweep" examples, the
 *    "AMD reducer constraint" paragraph and the "Tunables" list.
 *  - Tile rule: AITER issue "[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the CU
 *    count", section "Why it is not monotonic in num_queries".
 *  - Attention: moonmath-amd README, "MLA decode" usage section (fused 576-wide fp8 rows that
 *    are both K and V, one per-tensor kv_scale, page_size 1 slot lists, draft position t
 *    attending KV [0, S - q_len + t]) and the gfx950 "forward_paged" description (K/V caches
 *    [pages, page_size, kv_heads, D] addressed through kv_indptr / kv_page_indices); the
 *    "Numerics" section fixes the comparison target as attention over the same dequantized KV.
 *  - Skipped keys: AITER issue "[Perf] pa_decode_sparse ...", section "Measurements" (the
 *    has_invalid flag of the top-k index lists): a negative slot id in an MLA index list is a
 *    key that is not attended.
 *  - bf16 cache: AITER issue "[Perf] pa_decode_sparse ...", closing paragraph (an offer to
 *    re-measure on a bf16 cache).  Read as the same fused rows stored as bf16 instead of fp8,
 *    dequantized by the same per-tensor scale (1 for a plain bf16 cache).
 *  - Second cache: FlashInfer API page "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits", Parameters
 *    (extra_topk: candidate slots per token in a second cache).  Read as a second pool of rows of
 *    the same format and scale whose candidates a query attends together with its main-cache
 *    candidates, in one softmax.
 *  - Merge: base-2 log-sum-exp combination of partial results, the operation behind
 *    mla_splitk_reduce ("AMD reducer constraint") and mla_dcp_lse_merge_ranks.
 *
 * Attention is computed exactly as its definition reads: for each row, all scores, their
 * maximum, the exponentials, their sum, the weighted sum of values -- in binary64, unsplit.
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------ */
/* Number formats                                                                              */
/* ------------------------------------------------------------------------------------------ */

/* E4M3: 1 sign bit, 4 exponent bits, 3 mantissa bits.
 * OCP e4m3fn: bias 7; exponent field 0 is subnormal (m/8 * 2^(1-7)); S.1111.111 is NaN; no inf.
 * e4m3fnuz:   bias 8; exponent field 0 is subnormal (m/8 * 2^(1-8)); only 0x80 is NaN (there is
 *             no negative zero); no inf. */
double oracle_e4m3_value(uint32_t byte, int fnuz) {
    byte &= 0xffu;
    const int sign = (byte >> 7) & 1;
    const int e = (byte >> 3) & 0xf;
    const int m = byte & 0x7;
    const int bias = fnuz ? 8 : 7;
    if (fnuz) {
        if (byte == 0x80u) return NAN;
    } else {
        if (e == 0xf && m == 0x7) return NAN;
    }
    double mag;
    if (e == 0)
        mag = ldexp((double)m / 8.0, 1 - bias);
    else
        mag = ldexp(1.0 + (double)m / 8.0, e - bias);
    return sign ? -mag : mag;
}

/* bfloat16 is the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint32_t bits) {
    uint32_t w = (bits & 0xffffu) << 16;
    float f;
    memcpy(&f, &w, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------------------------ */
/* Planner                                                                                     */
/* ------------------------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
static int64_t max64(int64_t a, int64_t b) { return a > b ? a : b; }

/* Smallest power of two >= x (x >= 1). */
static int64_t next_pow2(int64_t x) {
    int64_t p = 1;
    while (p < x) p *= 2;
    return p;
}

/* Steps, in the page's order:
 *  1. Tunables: BM = 32 queries per MLA CTA; SPLIT_PAGE_SIZE = 256 keys (128 for single-kv-head
 *     MHA); MAX_PAGES_PER_SPLIT = 5; partition cap 256 for MLA-style (the reducer's limit),
 *     64 for MHA-style, narrowed to 32 at exactly 16 kv heads from batch 8 up.
 *  2. Regime: MLA-style when the caller is the MLA path or heads_per_group >= BM, else MHA-style.
 *  3. CTAs per partition: ceildiv(heads_per_group, BM) * batch (MLA-style) or
 *     heads_per_group * batch (MHA-style).
 *  4. one_wave = sm // ctas, two_wave = 2 * sm // ctas (read left to right),
 *     work_floor = ceildiv(pages, MAX_PAGES_PER_SPLIT), pages = ceildiv(num_keys, page size).
 *  5. Target: the two-wave exception min(two_wave, pages) for MLA with <= 16 heads and for
 *     single-kv-head MHA; for MHA-style when one unsplit wave already fills the device, the
 *     page asks only for enough partitions to amortize the key reads and prints no formula --
 *     work_floor is the reading adopted here; otherwise clamp(work_floor, one_wave, two_wave).
 *  6. Bucket up to the next power of two (the Phase-0 sweep rounds a work floor of 103 to 128).
 *  7. Cap, then the page floor (never more partitions than pages), and at least 1. */
int64_t oracle_plan_splits(int64_t batch_size, int64_t num_keys, int64_t heads_per_group,
                           int64_t sm_count, int is_mla) {
    if (batch_size <= 0 || heads_per_group <= 0 || sm_count <= 0 || num_keys < 0) return -1;

    const int64_t BM = 32;
    const int64_t MAX_PAGES_PER_SPLIT = 5;

    const int mla_style = is_mla || heads_per_group >= BM;
    const int64_t split_page_size = (!mla_style && heads_per_group == 1) ? 128 : 256;
    const int64_t pages = ceil_div(num_keys, split_page_size);

    int64_t ctas, cap;
    if (mla_style) {
        ctas = ceil_div(heads_per_group, BM) * batch_size;
        cap = 256;
    } else {
        ctas = heads_per_group * batch_size;
        cap = (heads_per_group == 16 && batch_size >= 8) ? 32 : 64;
    }

    const int64_t one_wave = sm_count / ctas;
    const int64_t two_wave = (2 * sm_count) / ctas;
    const int64_t work_floor = ceil_div(pages, MAX_PAGES_PER_SPLIT);

    int64_t target;
    const int exception = (is_mla && heads_per_group <= 16) || (!mla_style && heads_per_group == 1);
    if (exception)
        target = min64(two_wave, pages);
    else if (!mla_style && ctas >= sm_count)
        target = work_floor;
    else
        target = min64(max64(work_floor, one_wave), two_wave);

    target = next_pow2(max64(target, 1));
    int64_t np = min64(min64(target, cap), pages);
    return max64(np, 1);
}

int oracle_block_k(int64_t ctas, int64_t sm_count) {
    if (ctas <= 0 || sm_count <= 0) return -1;
    return ctas > sm_count ? 32 : 64;
}

/* Sparse top-k split planner (FlashInfer API page "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits",
 * the measured split rules and the GB10 paragraph), in the page's order:
 *  1. Work: candidates in chunks of 64, counted per cache (a chunk holds one cache's slots);
 *     CTAs of 16 * head_tiles heads, so the unsplit grid is num_tokens * ceil(heads / that).
 *  2. Two chunks (or fewer) never split.
 *  3. While the unsplit grid covers at most 40 % of the SMs, the largest power-of-two split
 *     (up to max_splits) whose grid stays within 80 % of the SMs and that leaves every CTA at
 *     least two chunks -- one chunk per CTA is allowed for a lone CTA only.
 *     Fewer than 64 SMs (the GB10 paragraph): the grid stays within SMs / 3 CTAs instead, the
 *     gather streams num_tokens * splits within SMs / 6, and two chunks per CTA hold for a lone
 *     CTA too.
 *  4. Once the unsplit grid fills the SMs, a split in two only for 16-chunk work whose doubled
 *     grid ends in a wave at least half full (not below 64 SMs: no wave-quantization split).
 *  5. Everything else unsplit.
 *  6. Independently, at most 16 chunks per CTA (the CTA index table): at least ceil(chunks / 16)
 *     splits, an error when max_splits is below that.
 *  7. chunks_per_block = ceil(chunks / num_splits).
 * Percentages are compared exactly in integers (10 * grid <= 4 * SMs, 10 * grid <= 8 * SMs). */
int oracle_plan_sparse_splits(int64_t num_tokens, int64_t num_heads, int64_t topk,
                              int64_t extra_topk, int64_t num_sms, int64_t max_splits,
                              int64_t head_tiles, int64_t *num_splits, int64_t *chunks_per_block) {
    if (num_tokens <= 0 || num_heads <= 0 || num_sms <= 0 || max_splits <= 0 || head_tiles <= 0 ||
        topk < 0 || extra_topk < 0 || !num_splits || !chunks_per_block)
        return -1;

    /* step 1 */
    const int64_t CHUNK = 64;
    const int64_t MAX_CHUNKS_PER_BLOCK = 16;
    const int64_t chunks = ceil_div(topk, CHUNK) + ceil_div(extra_topk, CHUNK);
    const int64_t grid = num_tokens * ceil_div(num_heads, 16 * head_tiles);
    const int small_device = num_sms < 64;

    int64_t splits = 1;
    if (chunks <= 2) {
        /* step 2 */
        splits = 1;
    } else if (10 * grid <= 4 * num_sms) {
        /* step 3 */
        const int lone = grid == 1 && !small_device;
        for (int64_t s = 1; s <= max_splits; s *= 2) {
            int ok;
            if (small_device)
                ok = grid * s <= num_sms / 3 && num_tokens * s <= num_sms / 6;
            else
                ok = 10 * grid * s <= 8 * num_sms;
            ok = ok && (lone ? chunks >= s : chunks >= 2 * s);
            if (ok) splits = s;
        }
    } else if (grid >= num_sms) {
        /* step 4 */
        if (!small_device && chunks == 16) {
            const int64_t last = (2 * grid) % num_sms;
            if (last == 0 || 2 * last >= num_sms) splits = 2;
        }
    }
    /* step 5: otherwise unsplit */

    /* step 6 */
    const int64_t forced = ceil_div(chunks, MAX_CHUNKS_PER_BLOCK);
    if (forced > max_splits) return -1;
    splits = max64(splits, forced);
    splits = min64(splits, max_splits);

    /* step 7 */
    *num_splits = splits;
    *chunks_per_block = chunks > 0 ? ceil_div(chunks, splits) : 0;
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Attention                                                                                   */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    /* common */
    int64_t q_len, H, dv;
    const int32_t *kv_indptr, *seq_lens;
    double scale;
    const int64_t *rows;
    int64_t n_rows;
    double *o_out, *lse2_out;
    int is_mla;
    /* MLA */
    int64_t d_lat, d_rope;
    const uint16_t *q_lat, *q_pe;
    const uint8_t *pool;
    const int32_t *kv_indices;
    double kv_scale;
    const uint8_t *pool2;            /* a second cache, or NULL */
    const int32_t *kv2_indices, *kv2_indptr;
    const double *fp8_table; /* 256 decoded values */
    int kv_bf16;             /* the pool holds bf16 rows (2 bytes per element) instead of fp8 */
    /* GQA */
    int64_t Hkv, D, page_size;
    const uint16_t *q, *k_cache, *v_cache;
    const int32_t *kv_page_indices;
    /* work split */
    int64_t first, last;
    int error;
} attn_job;

/* Keys row (b, t) sees: the end-aligned draft window, then (q_len 1 only) every candidate of
 * the second cache. */
static int64_t keys_seen(const attn_job *j, int64_t b, int64_t t) {
    int64_t L = (int64_t)j->seq_lens[b] - j->q_len + t + 1;
    if (L < 0) L = 0;
    if (j->pool2) L += j->kv2_indptr[b + 1] - j->kv2_indptr[b];
    return L;
}

/* Row of key k of request b: main-cache keys first, then the second cache's; NULL for a
 * skipped key (a negative slot id). */
static const uint8_t *mla_row(const attn_job *j, int64_t b, int64_t k) {
    const int64_t dqk = j->d_lat + j->d_rope;
    int64_t slot;
    const uint8_t *pool;
    if (!j->pool2 || k < j->seq_lens[b]) {
        slot = j->kv_indices[j->kv_indptr[b] + k];
        pool = j->pool;
    } else {
        slot = j->kv2_indices[j->kv2_indptr[b] + (k - j->seq_lens[b])];
        pool = j->pool2;
    }
    return slot < 0 ? NULL : pool + slot * dqk * (j->kv_bf16 ? 2 : 1);
}

/* Element d of a pool row, dequantized: e4m3 by table, or bf16, times kv_scale. */
static double mla_elem(const attn_job *j, const uint8_t *row, int64_t d) {
    const double x = j->kv_bf16 ? oracle_bf16_value(((const uint16_t *)row)[d]) : j->fp8_table[row[d]];
    return x * j->kv_scale;
}

/* Scores s[0..L) of one MLA row against its keys. */
static void mla_scores(const attn_job *j, int64_t r, int64_t b, int64_t L, double *s,
                       double *qv) {
    const int64_t dqk = j->d_lat + j->d_rope;
    for (int64_t d = 0; d < j->d_lat; ++d) qv[d] = oracle_bf16_value(j->q_lat[r * j->d_lat + d]);
    for (int64_t d = 0; d < j->d_rope; ++d)
        qv[j->d_lat + d] = oracle_bf16_value(j->q_pe[r * j->d_rope + d]);
    for (int64_t k = 0; k < L; ++k) {
        const uint8_t *row = mla_row(j, b, k);
        if (!row) {   /* a skipped key: no weight */
            s[k] = -INFINITY;
            continue;
        }
        double dot = 0.0;
        for (int64_t d = 0; d < dqk; ++d) dot += qv[d] * mla_elem(j, row, d);
        s[k] = j->scale * dot;
    }
}

static double mla_value(const attn_job *j, int64_t b, int64_t k, int64_t d) {
    return mla_elem(j, mla_row(j, b, k), d);
}

static const uint16_t *gqa_row(const attn_job *j, const uint16_t *cache, int64_t b, int64_t k,
                               int64_t kvh) {
    const int64_t page = j->kv_page_indices[j->kv_indptr[b] + k / j->page_size];
    const int64_t slot = k % j->page_size;
    return cache + ((page * j->page_size + slot) * j->Hkv + kvh) * j->D;
}

static void gqa_scores(const attn_job *j, int64_t r, int64_t b, int64_t h, int64_t L, double *s,
                       double *qv) {
    const int64_t kvh = h / (j->H / j->Hkv);
    for (int64_t d = 0; d < j->D; ++d) qv[d] = oracle_bf16_value(j->q[r * j->D + d]);
    for (int64_t k = 0; k < L; ++k) {
        const uint16_t *krow = gqa_row(j, j->k_cache, b, k, kvh);
        double dot = 0.0;
        for (int64_t d = 0; d < j->D; ++d) dot += qv[d] * oracle_bf16_value(krow[d]);
        s[k] = j->scale * dot;
    }
}

static void *attn_worker(void *arg) {
    attn_job *j = (attn_job *)arg;
    const int64_t dq = j->is_mla ? (j->d_lat + j->d_rope) : j->D;
    int64_t max_L = 0;
    for (int64_t i = j->first; i < j->last; ++i) {
        const int64_t r = j->rows ? j->rows[i] : i;
        const int64_t b = r / (j->q_len * j->H);
        const int64_t t = (r / j->H) % j->q_len;
        const int64_t L = keys_seen(j, b, t);
        if (L > max_L) max_L = L;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)(max_L > 0 ? max_L : 1));
    double *qv = (double *)malloc(sizeof(double) * (size_t)dq);
    double *acc = (double *)malloc(sizeof(double) * (size_t)j->dv);
    if (!s || !qv || !acc) {
        j->error = 1;
        free(s); free(qv); free(acc);
        return NULL;
    }
    for (int64_t i = j->first; i < j->last; ++i) {
        const int64_t r = j->rows ? j->rows[i] : i;
        const int64_t b = r / (j->q_len * j->H);
        const int64_t t = (r / j->H) % j->q_len;
        const int64_t h = r % j->H;
        const int64_t L = keys_seen(j, b, t);
        double *o = j->o_out + i * j->dv;
        if (L == 0) {
            for (int64_t d = 0; d < j->dv; ++d) o[d] = 0.0;
            j->lse2_out[i] = -INFINITY;
            continue;
        }
        if (j->is_mla)
            mla_scores(j, r, b, L, s, qv);
        else
            gqa_scores(j, r, b, h, L, s, qv);

        /* softmax(s) . V, with the maximum subtracted before exponentiation */
        double m = s[0];
        for (int64_t k = 1; k < L; ++k)
            if (s[k] > m) m = s[k];
        if (m == -INFINITY) {   /* every key skipped: as if the row saw none */
            for (int64_t d = 0; d < j->dv; ++d) o[d] = 0.0;
            j->lse2_out[i] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t d = 0; d < j->dv; ++d) acc[d] = 0.0;
        for (int64_t k = 0; k < L; ++k) {
            if (s[k] == -INFINITY) continue;   /* a skipped key */
            const double p = exp(s[k] - m);
            l += p;
            if (j->is_mla) {
                for (int64_t d = 0; d < j->dv; ++d) acc[d] += p * mla_value(j, b, k, d);
            } else {
                const uint16_t *vrow = gqa_row(j, j->v_cache, b, k, h / (j->H / j->Hkv));
                for (int64_t d = 0; d < j->dv; ++d) acc[d] += p * oracle_bf16_value(vrow[d]);
            }
        }
        for (int64_t d = 0; d < j->dv; ++d) o[d] = acc[d] / l;
        /* log2 of sum_k e^{s_k} */
        j->lse2_out[i] = (m + log(l)) / log(2.0);
    }
    free(s); free(qv); free(acc);
    return NULL;
}

int oracle_default_threads(void) {
    cpu_set_t set;
    if (sched_getaffinity(0, sizeof set, &set) == 0) {
        int n = CPU_COUNT(&set);
        if (n > 0) return n;
    }
    return 1;
}

static int run_jobs(attn_job *proto, int n_threads) {
    if (n_threads <= 0) n_threads = oracle_default_threads();
    if (n_threads > proto->n_rows) n_threads = (int)(proto->n_rows > 0 ? proto->n_rows : 1);
    attn_job *jobs = (attn_job *)calloc((size_t)n_threads, sizeof(attn_job));
    pthread_t *tids = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !tids) { free(jobs); free(tids); return -1; }
    /* interleave rows over threads in contiguous chunks */
    const int64_t per = (proto->n_rows + n_threads - 1) / n_threads;
    int started = 0, rc = 0;
    for (int i = 0; i < n_threads; ++i) {
        jobs[i] = *proto;
        jobs[i].first = (int64_t)i * per;
        jobs[i].last = min64(proto->n_rows, jobs[i].first + per);
        if (jobs[i].first >= jobs[i].last) break;
        if (pthread_create(&tids[i], NULL, attn_worker, &jobs[i]) != 0) { rc = -1; break; }
        ++started;
    }
    for (int i = 0; i < started; ++i) {
        pthread_join(tids[i], NULL);
        if (jobs[i].error) rc = -1;
    }
    free(jobs); free(tids);
    return rc;
}

/* Validates the row list and the per-request key ranges against the index list sizes. */
static int check_rows(const int64_t *rows, int64_t n_rows, int64_t total_rows) {
    if (n_rows < 0) return -1;
    if (rows)
        for (int64_t i = 0; i < n_rows; ++i)
            if (rows[i] < 0 || rows[i] >= total_rows) return -1;
    if (!rows && n_rows != total_rows) return -1;
    return 0;
}

static int mla_decode(int64_t B, int64_t q_len, int64_t H, int64_t d_lat, int64_t d_rope,
                      int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                      const uint8_t *pool, int64_t pool_rows, const int32_t *kv_indices,
                      const int32_t *kv_indptr, const int32_t *seq_lens,
                      const uint8_t *pool2, int64_t pool2_rows, const int32_t *kv2_indices,
                      const int32_t *kv2_indptr, double scale,
                      double kv_scale, int fnuz, int kv_bf16, const int64_t *rows, int64_t n_rows,
                      double *o_out, double *lse2_out, int n_threads) {
    if (B <= 0 || q_len <= 0 || H <= 0 || d_lat <= 0 || d_rope < 0 || d_v <= 0) return -1;
    if (pool2) {
        if (q_len != 1 || !kv2_indices || !kv2_indptr) return -1;
        for (int64_t b = 0; b < B; ++b) {
            if (kv2_indptr[b + 1] < kv2_indptr[b]) return -1;
            for (int64_t k = kv2_indptr[b]; k < kv2_indptr[b + 1]; ++k)
                if (kv2_indices[k] >= pool2_rows) return -1;   /* negative: a skipped key */
        }
    }
    if (d_v > d_lat + d_rope) return -1;
    if (!q_lat || (d_rope > 0 && !q_pe) || !pool || !kv_indices || !kv_indptr || !seq_lens ||
        !o_out || !lse2_out)
        return -1;
    if (check_rows(rows, n_rows, B * q_len * H)) return -1;
    for (int64_t b = 0; b < B; ++b) {
        if (seq_lens[b] < 0 || kv_indptr[b + 1] - kv_indptr[b] < seq_lens[b]) return -1;
        for (int64_t k = 0; k < seq_lens[b]; ++k) {
            const int32_t slot = kv_indices[kv_indptr[b] + k];
            if (slot >= pool_rows) return -1;   /* negative: a skipped key */
        }
    }
    double table[256];
    for (int i = 0; i < 256; ++i) table[i] = oracle_e4m3_value((uint32_t)i, fnuz);

    attn_job proto;
    memset(&proto, 0, sizeof proto);
    proto.is_mla = 1;
    proto.q_len = q_len; proto.H = H; proto.dv = d_v;
    proto.kv_indptr = kv_indptr; proto.seq_lens = seq_lens;
    proto.scale = scale; proto.rows = rows; proto.n_rows = n_rows;
    proto.o_out = o_out; proto.lse2_out = lse2_out;
    proto.d_lat = d_lat; proto.d_rope = d_rope; proto.q_lat = q_lat; proto.q_pe = q_pe;
    proto.pool = pool; proto.kv_indices = kv_indices; proto.kv_scale = kv_scale;
    proto.pool2 = pool2; proto.kv2_indices = kv2_indices; proto.kv2_indptr = kv2_indptr;
    proto.fp8_table = table;
    proto.kv_bf16 = kv_bf16;
    if (n_rows == 0) return 0;
    return run_jobs(&proto, n_threads);
}

int oracle_mla_decode(int64_t B, int64_t q_len, int64_t H, int64_t d_lat, int64_t d_rope,
                      int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                      const uint8_t *pool, int64_t pool_rows, const int32_t *kv_indices,
                      const int32_t *kv_indptr, const int32_t *seq_lens, double scale,
                      double kv_scale, int fnuz, const int64_t *rows, int64_t n_rows,
                      double *o_out, double *lse2_out, int n_threads) {
    return mla_decode(B, q_len, H, d_lat, d_rope, d_v, q_lat, q_pe, pool, pool_rows, kv_indices,
                      kv_indptr, seq_lens, NULL, 0, NULL, NULL, scale, kv_scale, fnuz, 0, rows,
                      n_rows, o_out, lse2_out, n_threads);
}

int oracle_mla_decode_bf16(int64_t B, int64_t q_len, int64_t H, int64_t d_lat, int64_t d_rope,
                           int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                           const uint16_t *pool, int64_t pool_rows, const int32_t *kv_indices,
                           const int32_t *kv_indptr, const int32_t *seq_lens, double scale,
                           double kv_scale, const int64_t *rows, int64_t n_rows, double *o_out,
                           double *lse2_out, int n_threads) {
    return mla_decode(B, q_len, H, d_lat, d_rope, d_v, q_lat, q_pe, (const uint8_t *)pool, pool_rows,
                      kv_indices, kv_indptr, seq_lens, NULL, 0, NULL, NULL, scale, kv_scale, 0, 1,
                      rows, n_rows, o_out, lse2_out, n_threads);
}

int oracle_mla_decode_two_caches(int64_t B, int64_t H, int64_t d_lat, int64_t d_rope,
                                 int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                                 const uint8_t *pool, int64_t pool_rows,
                                 const int32_t *kv_indices, const int32_t *kv_indptr,
                                 const int32_t *seq_lens, const uint8_t *pool2,
                                 int64_t pool2_rows, const int32_t *kv2_indices,
                                 const int32_t *kv2_indptr, double scale, double kv_scale,
                                 const int64_t *rows, int64_t n_rows, double *o_out,
                                 double *lse2_out, int n_threads) {
    if (!pool2) return -1;
    return mla_decode(B, 1, H, d_lat, d_rope, d_v, q_lat, q_pe, pool, pool_rows, kv_indices,
                      kv_indptr, seq_lens, pool2, pool2_rows, kv2_indices, kv2_indptr, scale,
                      kv_scale, 0, 0, rows, n_rows, o_out, lse2_out, n_threads);
}

/* The second cache over a bf16 pool: both caches hold bf16 rows of the same width and scale. */
int oracle_mla_decode_two_caches_bf16(int64_t B, int64_t H, int64_t d_lat, int64_t d_rope,
                                      int64_t d_v, const uint16_t *q_lat, const uint16_t *q_pe,
                                      const uint16_t *pool, int64_t pool_rows,
                                      const int32_t *kv_indices, const int32_t *kv_indptr,
                                      const int32_t *seq_lens, const uint16_t *pool2,
                                      int64_t pool2_rows, const int32_t *kv2_indices,
                                      const int32_t *kv2_indptr, double scale, double kv_scale,
                                      const int64_t *rows, int64_t n_rows, double *o_out,
                                      double *lse2_out, int n_threads) {
    if (!pool2) return -1;
    return mla_decode(B, 1, H, d_lat, d_rope, d_v, q_lat, q_pe, (const uint8_t *)pool, pool_rows,
                      kv_indices, kv_indptr, seq_lens, (const uint8_t *)pool2, pool2_rows,
                      kv2_indices, kv2_indptr, scale, kv_scale, 0, 1, rows, n_rows, o_out,
                      lse2_out, n_threads);
}

int oracle_gqa_decode(int64_t B, int64_t q_len, int64_t Hq, int64_t Hkv, int64_t D,
                      int64_t page_size, const uint16_t *q, const uint16_t *k_cache,
                      const uint16_t *v_cache, int64_t num_pages,
                      const int32_t *kv_page_indices, const int32_t *kv_indptr,
                      const int32_t *seq_lens, double scale, const int64_t *rows,
                      int64_t n_rows, double *o_out, double *lse2_out, int n_threads) {
    if (B <= 0 || q_len <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || page_size <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (!q || !k_cache || !v_cache || !kv_page_indices || !kv_indptr || !seq_lens || !o_out ||
        !lse2_out)
        return -1;
    if (check_rows(rows, n_rows, B * q_len * Hq)) return -1;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t n_pages_b = kv_indptr[b + 1] - kv_indptr[b];
        if (seq_lens[b] < 0 || n_pages_b * page_size < seq_lens[b]) return -1;
        for (int64_t p = 0; p < ceil_div(seq_lens[b], page_size); ++p) {
            const int32_t page = kv_page_indices[kv_indptr[b] + p];
            if (page < 0 || page >= num_pages) return -1;
        }
    }
    attn_job proto;
    memset(&proto, 0, sizeof proto);
    proto.is_mla = 0;
    proto.q_len = q_len; proto.H = Hq; proto.dv = D;
    proto.kv_indptr = kv_indptr; proto.seq_lens = seq_lens;
    proto.scale = scale; proto.rows = rows; proto.n_rows = n_rows;
    proto.o_out = o_out; proto.lse2_out = lse2_out;
    proto.Hkv = Hkv; proto.D = D; proto.page_size = page_size;
    proto.q = q; proto.k_cache = k_cache; proto.v_cache = v_cache;
    proto.kv_page_indices = kv_page_indices;
    if (n_rows == 0) return 0;
    return run_jobs(&proto, n_threads);
}

/* ------------------------------------------------------------------------------------------ */
/* Merge                                                                                       */
/* ------------------------------------------------------------------------------------------ */

int oracle_lse_merge(int64_t rows, int64_t np, int64_t dv, const double *partial_o,
                     const double *partial_lse2, double *o_out, double *lse2_out) {
    if (rows < 0 || np <= 0 || dv <= 0 || !partial_o || !partial_lse2 || !o_out || !lse2_out)
        return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *lp = partial_lse2 + r * np;
        double m = -INFINITY;
        for (int64_t p = 0; p < np; ++p)
            if (lp[p] > m) m = lp[p];
        double *o = o_out + r * dv;
        for (int64_t d = 0; d < dv; ++d) o[d] = 0.0;
        if (m == -INFINITY) {
            lse2_out[r] = -INFINITY;
            continue;
        }
        /* sum_p 2^lse2_p, factored as 2^m * sum_p 2^(lse2_p - m) */
        double sum = 0.0;
        for (int64_t p = 0; p < np; ++p)
            if (lp[p] != -INFINITY) sum += exp2(lp[p] - m);
        const double lse2 = m + log2(sum);
        for (int64_t p = 0; p < np; ++p) {
            if (lp[p] == -INFINITY) continue;
            const double w = exp2(lp[p] - lse2);
            const double *op = partial_o + (r * np + p) * dv;
            for (int64_t d = 0; d < dv; ++d) o[d] += w * op[d];
        }
        lse2_out[r] = lse2;
    }
    return 0;
}
