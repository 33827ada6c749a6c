// gqa_split.hip -- split kernel of grouped-query decode over bf16 K/V pages, gfx950.
//
// What it computes (moonmath-amd README, gfx950 "forward_paged": caches
// [pages, page_size, kv_heads, 128], kv_indptr counting pages per sequence, kv_page_indices;
// Modular MAX planner page, MHA-style bullet: one CTA per (kv head, request) per partition):
// for one kv head of one request and one partition of its tokens, the query rows of that head
// group (q_len x group <= 64 of them) attend the partition's tokens; the CTA writes each row's
// softmax-weighted mean of values and the base-2 log-sum-exp of its scores.
//
// Layout of the work: one wave per 16 query rows.  Up to 16 rows per kv head the CTA is one wave
// and has no barriers; 17 to 32 rows take W = 2 waves, wave w holding rows 16 w .. 16 w + 15,
// both reading the same K and V tiles from LDS, with one barrier per tile.  With an even number of
// kv heads and up to 16 rows per head, gqa_pair_kernel below runs instead: one CTA per two kv
// heads, one wave each, copying both heads' rows of a token as one 512-byte run; 33 to 64 rows
// run on gqa_rows32_kernel (two waves of 32 rows, 32-token tiles).  At 16 rows this path
// reads 8 flop per byte, so it only has to keep HBM busy: the CTA streams its tokens in tiles of
// 16 through a ring of three LDS slots, each tile's K and V rows (256 bytes per token) copied
// straight from HBM into LDS with global_load_lds_dwordx4 (the W waves share the copies); tile
// t + 2 is issued before tile t is computed.  The small ring (24 KiB) lets six one-wave CTAs
// share a CU; on MI355X more waves with shallower rings move more bytes than fewer with deeper
// ones.  The copies are issued from inline assembly and waited for with explicit vmcnt counts
// (the compiler would drain every copy before each LDS read); page ids come through scalar
// loads, which count on a different counter.
//   - QK^T on v_mfma_f32_16x16x32_bf16 as S^T = K Q^T: the query rows are the 16 B-operand
//     columns (unused columns are zero); lane (row, g) then holds the scores of tokens 4g..4g+3.
//   - PV on v_mfma_f32_16x16x16_bf16 as O^T = V^T P^T: those four probabilities are exactly the
//     lane's B operand, and ds_read_b64_tr_b16 hands each lane 4 tokens of one value column.
//
// Order of the CTAs: CTAs share no data, so they are dispatched in plain order, which deals them
// round-robin over the 8 XCDs and gives each XCD an equal share of every request.  A CTA's work
// is proportional to its request's length, so (for batches of up to 64 requests) requests are
// taken longest first: the CTAs that start last are the shortest, and the grid drains evenly.
//
// LDS slot layout: token t's 256-byte row at t * 256, its 16-byte chunk c at chunk position
// c ^ swz(t) with swz a permutation of the 4 token bits.  Score-operand reads (16 tokens, one
// chunk) and transposed value reads (4 tokens x 2 chunks) are free of bank conflicts.
#include "device_common.hpp"
#include "kernels.hpp"

namespace gqa {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kD = 128;
constexpr int kTile = 16;        // tokens per tile
constexpr int kSlots = 3;        // LDS ring
constexpr int kRowBytes = kD * 2;
constexpr int kSlotBytes = 2 * kTile * kRowBytes;   // K then V

__device__ __forceinline__ int swz(int t) {
    return ((t & 3) << 1) | ((t >> 2) & 1) | (t & 8);
}
// Byte offset, inside a K or V block, of 16-byte chunk c of tile token t.
__device__ __forceinline__ int vpos(int t, int c) { return t * kRowBytes + ((c ^ swz(t)) << 4); }

// The fp32 partial rows (the reducer reads each once) are stored non-temporal.  Each store
// instruction covers 64 bytes of 8 or 16 rows; with ordinary stores they cost 12 to 14 % of a
// split's time on MI355X at 1.5 % of its bytes, marked non-temporal about half of that.  (The
// 4-byte log-sum-exp stores are faster left ordinary.)
__device__ __forceinline__ void store_partial(f32x4 *p, f32x4 v) { __builtin_nontemporal_store(v, p); }

// Direct HBM -> LDS copy of 16 bytes per lane (lane L -> m0 + 16 L), non-temporal: each page is
// read once, and the streaming hint raises gfx950's read bandwidth.
__device__ __forceinline__ void copy16(const void *g, uint32_t m0) {
    asm volatile("global_load_lds_dwordx4 %0, off nt" ::"v"(g), "{m0}"(m0) : "memory");
}
// s_waitcnt vmcnt(n) for a wave-uniform n: the copies of `later` younger tiles (2 C copy
// instructions each, C copy steps per block and wave) may still be in flight.
template <int C>
__device__ __forceinline__ void wait_tiles(int later) {
    static_assert(kSlots == 3, "wait_tiles covers up to two younger tiles");
    if (later >= 2) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * C) : "memory");
    else if (later == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * C) : "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ float rows4_max(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The request of rank r when the batch is ordered by decreasing length (ties by index), for
// batches of up to 64 requests (lane i ranks request i); larger batches keep their own order.
__device__ __forceinline__ int request_by_length(const int32_t *seq_lens, int batch, int r, int lane) {
    if (batch > 64) return r;
    const int si = lane < batch ? seq_lens[lane] : -1;
    int rank = 0;
    for (int j = 0; j < batch; ++j) {
        const int sj = __builtin_amdgcn_readlane(si, j);
        rank += (sj > si) | ((sj == si) & (j < lane));
    }
    // ranks are a permutation of 0 .. batch - 1, so exactly one lane matches r < batch
    const uint64_t m = __builtin_amdgcn_ballot_w64(lane < batch && rank == r);
    return __builtin_amdgcn_readfirstlane(int(__builtin_ctzll(m)));
}

// One 16-token tile for one wave's 16 query rows (lane (col, g): row col, tokens 4 g .. 4 g + 3):
// S^T = K Q^T, the online softmax in base 2 (masking tokens at or past row_end when the tile
// reaches past kfull, the tokens every row sees), then O^T += V^T P^T.  k_off: this lane's score
// operand offsets in the K block kt; voff(j): its transposed read of value block j in vt.
template <typename VOff>
__device__ __forceinline__ void tile_math(const uint8_t *kt, const uint8_t *vt, const int (&k_off)[4], VOff voff,
                                          const bf16x8 (&qf)[4], float score_scale, int tb, int kfull,
                                          int row_end, int g, float &m_run, float &l_run, f32x4 (&oacc)[8]) {
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const u32x4 *>(kt + k_off[s])), qf[s], sacc, 0, 0, 0);

    // Online softmax in base 2; lane (col, g) holds tokens tb + 4 g + i of its row.
    float sv[4];
    const bool masked = tb + kTile > kfull;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sv[i] = sacc[i] * score_scale;
        if (masked && tb + 4 * g + i >= row_end) sv[i] = kNegInf;
    }
    const float mx = rows4_max(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(sv[i] - m_use);
    l_run = l_run * alpha + rows4_sum((p[0] + p[1]) + (p[2] + p[3]));
    m_run = m_new;
    if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[j] *= alpha;
    }
    // The weights go to the bf16 MFMA as two parts, p = hi + lo (hi = p rounded to bf16, lo = the
    // remainder rounded to bf16), so each carries a relative error of at most 2^-17 instead of
    // bf16's 2^-9 (which, with values of magnitude 16, alone moves the output by 0.03).  Both
    // parts go through one v_mfma_f32_16x16x32_bf16: the lane's k slots 8 g .. 8 g + 3 take V's
    // tokens 4 g .. 4 g + 3 against hi, slots 8 g + 4 .. 8 g + 7 the same tokens against lo.
    const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
    const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
    const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
    const bf16x8 pb = as_bf16x8(u32x4{h01, h23, l01, l23});
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x2 va = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4 *)(vt + voff(j))));
        oacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(u32x4{va[0], va[1], va[0], va[1]}), pb,
                                                          oacc[j], 0, 0, 0);
    }
}

template <bool DIRECT, int W>
__global__ void __launch_bounds__(64 * W) gqa_split_kernel(const GqaSplitArgs a) {
    // Two-wave CTAs reserve 40 KiB (16 KiB beyond the ring, holding nothing), which caps the CU at
    // four of them (eight waves) instead of six: on MI355X q_len 4 over 8 kv heads (32 rows per
    // kv head) ran 409-415 us per split against 430 us with six, 421 us with five, and fell to
    // 567-648 us with three or two.
    __shared__ __attribute__((aligned(1024))) uint8_t lds[kSlots * kSlotBytes + (W > 1 ? 16384 : 0)];

    const int logical = blockIdx.x;
    if (logical >= a.total_ctas) return;
    const int lane = W > 1 ? threadIdx.x & 63 : threadIdx.x, g = lane >> 4, col = lane & 15;
    const int wv = W > 1 ? __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6) : 0;
    const int kvh = logical % a.Hkv;
    const int rest = logical / a.Hkv;
    // np equal partitions per request (longest requests first), or the planned
    // length-proportional slots
    const int b = a.part_start ? request_of_slot(a.part_start, a.batch, rest)
                               : request_by_length(a.seq_lens, a.batch, rest / a.np, lane);
    if (b >= a.batch) return;
    const int part = a.part_start ? rest - a.part_start[b] : rest % a.np;
    const int rows_cta = a.q_len * a.group;
    const int page_mask = (1 << a.page_shift) - 1;

    // Tokens of this partition: ceil(S / np) rounded up to block_k (a multiple of the tile), the
    // last ones possibly empty; no row sees past the latest draft token.
    const int S = a.seq_lens[b];
    const int pbase = a.kv_indptr[b];
    const int chunk = a.part_start ? a.part_chunk[b]
                                   : ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int k1 = min(max(0, S - a.q_len + (rows_cta - 1) / a.group + 1), k0 + chunk);
    const int kfull = min(k1, max(0, S - a.q_len + 1));   // tokens every row sees
    const int ntiles = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;

    // Query row 16 wv + col of the group in MFMA column `col` of this wave.
    const int r = 16 * wv + col;
    const bool row_ok = r < rows_cta;
    const int t = row_ok ? r / a.group : 0;
    const int head = kvh * a.group + (row_ok ? r - t * a.group : 0);
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;

    bf16x8 qf[4];  // B operand: row 16 wv + col, d = 32 s + 8 g .. +7
    {
        const uint16_t *q = a.q + (int64_t(b) * a.q_len + t) * a.q_st_tok + int64_t(head) * a.q_st_head;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qf[s] = as_bf16x8(row_ok ? *reinterpret_cast<const u32x4 *>(q + 32 * s + 8 * g)
                                     : u32x4{0u, 0u, 0u, 0u});
    }

    // ---- copies.  Copy i of a block moves tokens 4i..4i+3: lane L carries token 4i + L/16 and
    // lands on chunk position L % 16 of its row, i.e. global chunk (L % 16) ^ swz(token).  Wave wv
    // issues copies 4 wv / W .. 4 (wv + 1) / W - 1 of each block.
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    const int64_t row_stride = int64_t(a.Hkv) * kRowBytes;       // bytes between tokens of a page
    const uint8_t *const kbase = reinterpret_cast<const uint8_t *>(a.k_cache) + int64_t(kvh) * kRowBytes;
    const uint8_t *const vbase = reinterpret_cast<const uint8_t *>(a.v_cache) + int64_t(kvh) * kRowBytes;
    // read-only, uniform: the constant address space makes these scalar loads
    typedef const __attribute__((address_space(4))) int32_t *const_ids;
    const const_ids pids = (const_ids)(uintptr_t)(a.page_indices + pbase);
    // Page ids of a tile (scalar loads): tokens tb..tb+15 lie on at most two pages.
    struct Pages { int p0, p1; };
    auto tile_pages = [&](int tile) -> Pages {
        const int tb = k0 + tile * kTile;
        const int last = min(tb + kTile, k1) - 1;
        return Pages{pids[tb >> a.page_shift], pids[last >> a.page_shift]};
    };
    constexpr int kCopies = 4 / W;   // copy steps per block and wave
    auto issue_tile = [&](int tile, Pages pg) {
        const int tb = k0 + tile * kTile;
        const int first_page_end = ((tb >> a.page_shift) + 1) << a.page_shift;
        const uint32_t m0 = lds_addr + (tile % kSlots) * kSlotBytes;
#pragma unroll
        for (int c = 0; c < kCopies; ++c) {
            const int i = kCopies * wv + c;
            const int tl = 4 * i + (lane >> 4);
            const int tok = min(tb + tl, k1 - 1);
            const int page = tok < first_page_end ? pg.p0 : pg.p1;
            const int64_t slot = (int64_t(page) << a.page_shift) | (tok & page_mask);
            const int64_t off = slot * row_stride + (((lane & 15) ^ swz(tl)) << 4);
            copy16(kbase + off, m0 + i * 1024);
            copy16(vbase + off, m0 + kTile * kRowBytes + i * 1024);
        }
    };

    // Loop-invariant LDS offsets: score operand (token col, chunk 4 s + g) and the transposed value
    // read (lane s = col of group g points at token 4 g + s / 4, columns 16 blk + 4 (s % 4)..+3,
    // i.e. chunk 2 blk + (s % 4) / 2, byte 8 (s % 2)).
    int k_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) k_off[s] = vpos(col, 4 * s + g);
    const int v_tok = 4 * g + (col >> 2);
    const int v_c = (col & 3) >> 1, v_b = 8 * (col & 1);

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    Pages next_pages{0, 0};
    if (ntiles > 0) {
#pragma unroll
        for (int j = 0; j < kSlots - 1; ++j)
            if (j < ntiles) issue_tile(j, tile_pages(j));
        if (kSlots - 1 < ntiles) next_pages = tile_pages(kSlots - 1);
    }
    // The queries are used from here on: the compiler waits for their loads (vmcnt(0), which
    // also covers the first two tiles' copies) once, here.  Without this use it would put that
    // wait at the first score of every tile, draining the copies of the tiles ahead each time,
    // which the multi-wave CTAs cannot afford.
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]));

    for (int it = 0; it < ntiles; ++it) {
        if (W == 1) {
            // slot (it + 2) % 3 held tile it - 1, whose reads all finished last iteration.  The
            // wave then waits for all its copies, tile it + 2's included: with six one-wave CTAs
            // per CU the other waves' copies keep HBM busy meanwhile, and on the 32-request paged
            // batch this ran 389 us per launch against 398 us when tiles it + 1 and it + 2 stay
            // in flight (measured on MI355X in one process).
            if (it + kSlots - 1 < ntiles) {
                issue_tile(it + kSlots - 1, next_pages);
                if (it + kSlots < ntiles) next_pages = tile_pages(it + kSlots);
            }
            wait_tiles<kCopies>(0);
        } else {
            // this wave's copies of tile it have landed; after the barrier so have every wave's,
            // and every wave is done reading tile it - 1, whose slot then takes tile it + 2
            wait_tiles<kCopies>(min(kSlots - 2, ntiles - 1 - it));
            __syncthreads();
            if (it + kSlots - 1 < ntiles) {
                issue_tile(it + kSlots - 1, next_pages);
                if (it + kSlots < ntiles) next_pages = tile_pages(it + kSlots);
            }
        }
        const uint8_t *kt = lds + (it % kSlots) * kSlotBytes;
        const uint8_t *vt = kt + kTile * kRowBytes;

        tile_math(kt, vt, k_off, [&](int j) { return vpos(v_tok, 2 * j + v_c) + v_b; }, qf, a.score_scale,
                  k0 + it * kTile, kfull, row_end, g, m_run, l_run, oacc);
    }

    // Lane (col, g) of block j holds value columns 16 j + 4 g .. + 3 of row 16 wv + col.
    if (!row_ok) return;
    const int64_t row = (int64_t(b) * a.q_len + t) * a.Hq + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    if (DIRECT) {
        uint16_t *o = a.out + row * kD + 4 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint2 *>(o + 16 * j) =
                make_uint2(pack_bf16x2(oacc[j][0] * inv, oacc[j][1] * inv),
                           pack_bf16x2(oacc[j][2] * inv, oacc[j][3] * inv));
        if (g == 0 && a.lse2_out) a.lse2_out[row] = lse2;
    } else {
        // partial row: [row, np] or, with planned slots, [slot, q_len * Hq]
        const int64_t prow = a.part_start ? (int64_t(rest) * a.q_len + t) * a.Hq + head
                                          : row * a.np + part;
        float *o = a.part_o + prow * kD + 4 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) store_partial(reinterpret_cast<f32x4 *>(o + 16 * j), oacc[j] * inv);
        if (g == 0) a.part_lse2[prow] = lse2;
    }
}

// ---- kv-head-pair variant, for an even number of kv heads and at most 16 query rows per head
// group.  A CTA serves HC = 2 consecutive kv heads of one (request, partition): wave w takes kv
// head h0 + w and its head group's query rows, as a one-wave CTA of gqa_split_kernel would.  A
// tile's 16 tokens of K (and of V) for those heads are 16 runs of HC x 256 contiguous bytes, and
// the CTA copies them as such: instruction i of thread tid moves the j-th 16-byte chunk,
// j = 64 HC i + tid, i.e. token j / (16 HC), head (j / 16) % HC, chunk position j % 16 (holding
// global chunk (j % 16) ^ swz(token)).  Measured on MI355X (32 requests, 8 kv heads, partial
// rows stored non-temporal): 2, 4 and 8 heads per CTA (8 = whole pages) within 3 % of each
// other, 2 the fastest and 2 % ahead of one-head CTAs; rings of 3 slots slower than 2.  The ring
// has two slots of HC x 16 KiB (five CTAs per CU); each step waits for this wave's copies of
// tile t, then a barrier (every copy landed, every wave done with tile t - 1), then the copies of
// tile t + 1 into tile t - 1's slot, then tile t's math.
constexpr int kPairSlots = 2;

template <bool DIRECT, int HC>
__global__ void __launch_bounds__(64 * HC) gqa_pair_kernel(const GqaSplitArgs a) {
    constexpr int kRow = HC * kRowBytes;            // one token's rows of the CTA's heads
    constexpr int kHalf = kTile * kRow;             // K (or V) part of a slot
    constexpr int SLOTS = kPairSlots;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[SLOTS * 2 * kHalf];

    const int logical = blockIdx.x;
    if (logical >= a.total_ctas) return;
    const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, col = lane & 15;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hgroups = a.Hkv / HC;
    const int h0 = (logical % hgroups) * HC;
    const int kvh = h0 + w;
    const int rest = logical / hgroups;
    const int b = a.part_start ? request_of_slot(a.part_start, a.batch, rest)
                               : request_by_length(a.seq_lens, a.batch, rest / a.np, lane);
    if (b >= a.batch) return;
    const int part = a.part_start ? rest - a.part_start[b] : rest % a.np;
    const int rows_cta = a.q_len * a.group;
    const int page_mask = (1 << a.page_shift) - 1;

    const int S = a.seq_lens[b];
    const int pbase = a.kv_indptr[b];
    const int chunk = a.part_start ? a.part_chunk[b]
                                   : ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int k1 = min(max(0, S - a.q_len + (rows_cta - 1) / a.group + 1), k0 + chunk);
    const int kfull = min(k1, max(0, S - a.q_len + 1));
    const int ntiles = k1 > k0 ? (k1 - k0 + kTile - 1) / kTile : 0;

    // query row col of kv head kvh's group
    const bool row_ok = col < rows_cta;
    const int t = row_ok ? col / a.group : 0;
    const int head = kvh * a.group + (row_ok ? col - t * a.group : 0);
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;
    bf16x8 qf[4];
    {
        const uint16_t *q = a.q + (int64_t(b) * a.q_len + t) * a.q_st_tok + int64_t(head) * a.q_st_head;
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qf[s] = as_bf16x8(row_ok ? *reinterpret_cast<const u32x4 *>(q + 32 * s + 8 * g)
                                     : u32x4{0u, 0u, 0u, 0u});
    }

    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    const int64_t row_stride = int64_t(a.Hkv) * kRowBytes;       // bytes between tokens of a page
    const uint8_t *const kbase = reinterpret_cast<const uint8_t *>(a.k_cache) + int64_t(h0) * kRowBytes;
    const uint8_t *const vbase = reinterpret_cast<const uint8_t *>(a.v_cache) + int64_t(h0) * kRowBytes;
    typedef const __attribute__((address_space(4))) int32_t *const_ids;
    const const_ids pids = (const_ids)(uintptr_t)(a.page_indices + pbase);
    struct Pages { int p0, p1; };
    auto tile_pages = [&](int tile) -> Pages {
        const int tb = k0 + tile * kTile;
        const int last = min(tb + kTile, k1) - 1;
        return Pages{pids[tb >> a.page_shift], pids[last >> a.page_shift]};
    };
    auto issue_tile = [&](int tile, Pages pg) {
        const int tb = k0 + tile * kTile;
        const int first_page_end = ((tb >> a.page_shift) + 1) << a.page_shift;
        const uint32_t m0 = lds_addr + (tile % SLOTS) * 2 * kHalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 64 * HC * i + tid;
            const int tl = j / (16 * HC), hh = (j >> 4) % HC;
            const int tok = min(tb + tl, k1 - 1);
            const int page = tok < first_page_end ? pg.p0 : pg.p1;
            const int64_t slot = (int64_t(page) << a.page_shift) | (tok & page_mask);
            const int64_t off = slot * row_stride + hh * kRowBytes + (((j & 15) ^ swz(tl)) << 4);
            copy16(kbase + off, m0 + 1024 * (HC * i + w));
            copy16(vbase + off, m0 + kHalf + 1024 * (HC * i + w));
        }
    };

    // this wave's reads: token tk's row of its head at tk * kRow + w * 256, chunks permuted
    auto posp = [&](int tk, int c) { return tk * kRow + w * kRowBytes + ((c ^ swz(tk)) << 4); };
    int k_off[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) k_off[s] = posp(col, 4 * s + g);
    const int v_tok = 4 * g + (col >> 2);
    const int v_c = (col & 3) >> 1, v_b = 8 * (col & 1);

    float m_run = kNegInf, l_run = 0.f;
    f32x4 oacc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) oacc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // tile 0 in flight before the loop; page ids one tile ahead of their copies
    static_assert(SLOTS == 2, "one tile in flight during the math");
    Pages next_pages{0, 0};
    if (ntiles > 0) issue_tile(0, tile_pages(0));
    if (1 < ntiles) next_pages = tile_pages(1);
    // (the queries are used here, so the compiler's wait for their loads is not inside the loop)
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]));

    for (int it = 0; it < ntiles; ++it) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's copies of tile it
        __syncthreads();   // tile it landed (every wave's copies); tile it - 1 read by every wave
        if (it + 1 < ntiles) {
            issue_tile(it + 1, next_pages);
            if (it + 2 < ntiles) next_pages = tile_pages(it + 2);
        }
        const uint8_t *kt = lds + (it % SLOTS) * 2 * kHalf;
        tile_math(kt, kt + kHalf, k_off, [&](int j) { return posp(v_tok, 2 * j + v_c) + v_b; }, qf,
                  a.score_scale, k0 + it * kTile, kfull, row_end, g, m_run, l_run, oacc);
    }

    if (!row_ok) return;
    const int64_t row = (int64_t(b) * a.q_len + t) * a.Hq + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    if (DIRECT) {
        uint16_t *o = a.out + row * kD + 4 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            *reinterpret_cast<uint2 *>(o + 16 * j) =
                make_uint2(pack_bf16x2(oacc[j][0] * inv, oacc[j][1] * inv),
                           pack_bf16x2(oacc[j][2] * inv, oacc[j][3] * inv));
        if (g == 0 && a.lse2_out) a.lse2_out[row] = lse2;
    } else {
        const int64_t prow = a.part_start ? (int64_t(rest) * a.q_len + t) * a.Hq + head
                                          : row * a.np + part;
        float *o = a.part_o + prow * kD + 4 * g;
#pragma unroll
        for (int j = 0; j < 8; ++j) store_partial(reinterpret_cast<f32x4 *>(o + 16 * j), oacc[j] * inv);
        if (g == 0) a.part_lse2[prow] = lse2;
    }
}

hipError_t launch_pair(const GqaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(a.total_ctas), block(64 * 2);
    if (direct)
        hipLaunchKernelGGL((gqa_pair_kernel<true, 2>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gqa_pair_kernel<false, 2>), grid, block, 0, s, a);
    return hipGetLastError();
}

// ---- 32-row variant, for 33 to 64 query rows per kv head (MQA, wide groups, draft windows).
// One CTA per (request, partition, kv head), two waves of 32 query rows, 32-token tiles on
// v_mfma_f32_32x32x16_bf16: per token and row it issues fewer instructions than 16-row waves
// (each K operand serves 32 rows, half the MFMAs, row reductions over 16 scores per lane).
// Measured on MI355X against four 16-row waves (64 query heads on one kv head, 32 requests of
// 1024 to 32768 tokens): 105 against 118 us at np = 16, 78 against 89-95 us at np = 64; q_len 8
// over 8 kv heads, 503-506 against 579-593 us.  A ring of 3 slots (3 CTAs per CU instead of 5)
// was slower, and so was one 32-row wave for 17 to 32 rows against two 16-row waves (451 against
// 431 us on q_len 4 over 8 kv heads), which keep that range.
//   - QK^T as S^T = K Q^T: MFMA s (0..7) covers dims 16 s .. 16 s + 15, lane (m, h) reading dims
//     16 s + 8 h .. + 7 of token m; lane (n, h) of the result holds row n's scores of tokens
//     8 j + 4 h + i (j, i = 0..3).
//   - PV as O^T = V^T P^T in K steps j = 0..3 of 16 slots: the lane's slots 8 h .. 8 h + 3 take
//     tokens 8 j + 4 h + 0..3 against the weights' bf16 hi parts, slots 8 h + 4 .. 8 h + 7 the same
//     tokens against the lo parts; ds_read_b64_tr_b16 hands lane (m, h) those 4 tokens of value
//     dim 32 mb + m (M block mb = 0..3).
//   - LDS: token t's 256-byte row at t * 256 in a 32-token K (then V) block, 16-byte chunk c at
//     position c ^ f(t), f(t) = ((t & 3) << 2) | ((t >> 2) & 3).  Score reads (one chunk of the 16
//     tokens a 16-lane read cycle serves) and transposed value reads (4 tokens x 4 chunks per
//     32-lane cycle) then touch distinct 16-byte (8-byte) slots of a bank row.
constexpr int kTile32 = 32;
constexpr int kHalf32 = kTile32 * kRowBytes;   // K (or V) block of a slot
constexpr int kSlots32 = 2;                    // LDS ring (32 KiB)
constexpr int kWaves32 = 2;
__device__ __forceinline__ int swz32(int t) { return ((t & 3) << 2) | ((t >> 2) & 3); }

template <bool DIRECT>
__global__ void __launch_bounds__(64 * kWaves32) gqa_rows32_kernel(const GqaSplitArgs a) {
    constexpr int W = kWaves32, SLOTS = kSlots32;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[SLOTS * 2 * kHalf32];
    typedef float f32x16 __attribute__((ext_vector_type(16)));

    const int logical = blockIdx.x;
    if (logical >= a.total_ctas) return;
    const int lane = threadIdx.x & 63;
    const int n = lane & 31, h = lane >> 5;
    const int wv = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6);
    const int kvh = logical % a.Hkv;
    const int rest = logical / a.Hkv;
    const int b = a.part_start ? request_of_slot(a.part_start, a.batch, rest)
                               : request_by_length(a.seq_lens, a.batch, rest / a.np, lane);
    if (b >= a.batch) return;
    const int part = a.part_start ? rest - a.part_start[b] : rest % a.np;
    const int rows_cta = a.q_len * a.group;
    const int page_mask = (1 << a.page_shift) - 1;

    const int S = a.seq_lens[b];
    const int pbase = a.kv_indptr[b];
    const int chunk = a.part_start ? a.part_chunk[b]
                                   : ((S + a.np - 1) / a.np + a.block_k - 1) / a.block_k * a.block_k;
    const int k0 = part * chunk;
    const int k1 = min(max(0, S - a.q_len + (rows_cta - 1) / a.group + 1), k0 + chunk);
    const int kfull = min(k1, max(0, S - a.q_len + 1));   // tokens every row sees
    const int ntiles = k1 > k0 ? (k1 - k0 + kTile32 - 1) / kTile32 : 0;

    // Query row 32 wv + n in MFMA column n of this wave.
    const int r = 32 * wv + n;
    const bool row_ok = r < rows_cta;
    const int t = row_ok ? r / a.group : 0;
    const int head = kvh * a.group + (row_ok ? r - t * a.group : 0);
    const int row_end = row_ok ? min(max(0, S - a.q_len + t + 1), k1) : k0;

    bf16x8 qf[8];  // B operand of QK MFMA s: row 32 wv + n, dims 16 s + 8 h .. + 7
    {
        const uint16_t *q = a.q + (int64_t(b) * a.q_len + t) * a.q_st_tok + int64_t(head) * a.q_st_head;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            qf[s] = as_bf16x8(row_ok ? *reinterpret_cast<const u32x4 *>(q + 16 * s + 8 * h)
                                     : u32x4{0u, 0u, 0u, 0u});
    }

    // ---- copies.  Instruction i (0..7) of a block moves tokens 4 i .. 4 i + 3: lane L carries
    // token 4 i + L / 16 and lands on chunk position L % 16 of its row, i.e. global chunk
    // (L % 16) ^ swz32(token).  Pages hold at least 8 tokens, so the 4 tokens of an instruction
    // share a page, whose id is one scalar load.  Wave wv issues instructions 8 wv / W ..
    const uint32_t lds_addr = uint32_t(reinterpret_cast<uintptr_t>(lds));
    const int64_t row_stride = int64_t(a.Hkv) * kRowBytes;
    const uint8_t *const kbase = reinterpret_cast<const uint8_t *>(a.k_cache) + int64_t(kvh) * kRowBytes;
    const uint8_t *const vbase = reinterpret_cast<const uint8_t *>(a.v_cache) + int64_t(kvh) * kRowBytes;
    typedef const __attribute__((address_space(4))) int32_t *const_ids;
    const const_ids pids = (const_ids)(uintptr_t)(a.page_indices + pbase);
    constexpr int kIns = 8 / W;   // copy instructions per block and wave
    struct Pages { int p[kIns]; };
    auto tile_pages = [&](int tile) -> Pages {
        const int tb = k0 + tile * kTile32;
        Pages pg;
#pragma unroll
        for (int c = 0; c < kIns; ++c) pg.p[c] = pids[min(tb + 4 * (kIns * wv + c), k1 - 1) >> a.page_shift];
        return pg;
    };
    auto issue_tile = [&](int tile, const Pages &pg) {
        const int tb = k0 + tile * kTile32;
        const uint32_t m0 = lds_addr + (tile % SLOTS) * 2 * kHalf32;
#pragma unroll
        for (int c = 0; c < kIns; ++c) {
            const int i = kIns * wv + c;
            const int tl = 4 * i + (lane >> 4);
            const int tok = min(tb + tl, k1 - 1);
            const int64_t slot = (int64_t(pg.p[c]) << a.page_shift) | (tok & page_mask);
            const int64_t off = slot * row_stride + (((lane & 15) ^ swz32(tl)) << 4);
            copy16(kbase + off, m0 + i * 1024);
            copy16(vbase + off, m0 + kHalf32 + i * 1024);
        }
    };

    // Loop-invariant LDS offsets.  Score operand of MFMA s: token n, chunk 2 s + h.  Transposed
    // value read of (M block mb, K step j): in 16-lane group (h, dh = bit 4 of the lane), lane
    // 4 k + e points at token 8 j + 4 h + k, dims 32 mb + 16 dh + 4 e .. + 3, i.e. chunk
    // 4 mb + 2 dh + e / 2, byte 8 (e % 2).
    const int dh = (lane >> 4) & 1, vk = (lane & 15) >> 2, ve = lane & 3;
    auto kpos = [&](int s) { return n * kRowBytes + (((2 * s + h) ^ swz32(n)) << 4); };
    auto vposj = [&](int mb, int j) {
        const int tk = 8 * j + 4 * h + vk;
        return tk * kRowBytes + (((4 * mb + 2 * dh + (ve >> 1)) ^ swz32(tk)) << 4) + 8 * (ve & 1);
    };

    float m_run = kNegInf, l_run = 0.f;
    f32x16 oacc[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[mb][i] = 0.f;

    Pages next_pages;
    if (ntiles > 0) issue_tile(0, tile_pages(0));
    if (1 < ntiles) next_pages = tile_pages(1);
    // (the queries are used here, so the compiler's wait for their loads is not inside the loop)
    asm volatile("" ::"v"(qf[0]), "v"(qf[1]), "v"(qf[2]), "v"(qf[3]), "v"(qf[4]), "v"(qf[5]), "v"(qf[6]),
                 "v"(qf[7]));

    static_assert(SLOTS == 2, "one tile in flight during the math");
    for (int it = 0; it < ntiles; ++it) {
        // this wave's copies of tile it have landed; after the barrier so have every wave's, and
        // every wave is done reading tile it - 1, whose slot then takes tile it + 1
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (it + 1 < ntiles) {
            issue_tile(it + 1, next_pages);
            if (it + 2 < ntiles) next_pages = tile_pages(it + 2);
        }
        const uint8_t *kt = lds + (it % SLOTS) * 2 * kHalf32;
        const uint8_t *vt = kt + kHalf32;
        const int tb = k0 + it * kTile32;

        f32x16 sacc;
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                as_bf16x8(*reinterpret_cast<const u32x4 *>(kt + kpos(s))), qf[s], sacc, 0, 0, 0);

        // online softmax in base 2; lane (n, h) holds tokens tb + 8 j + 4 h + i of row n
        float sv[16];
        const bool masked = tb + kTile32 > kfull;
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float x = sacc[4 * j + i] * a.score_scale;
                if (masked && tb + 8 * j + 4 * h + i >= row_end) x = kNegInf;
                sv[4 * j + i] = x;
                mx = fmaxf(mx, x);
            }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        const float m_new = fmaxf(m_run, mx);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            sv[i] = fast_exp2(sv[i] - m_use);
            psum += sv[i];
        }
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(psum), __float_as_uint(psum), false, false);
            psum = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (__builtin_amdgcn_ballot_w64(alpha != 1.f)) {
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) oacc[mb] *= alpha;
        }
        // weights as bf16 hi + lo (relative error at most 2^-17); K step j: {hi, lo} of tokens
        // 8 j + 4 h + 0..3
        bf16x8 pb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float *p = sv + 4 * j;
            const uint32_t h01 = pack_bf16x2(p[0], p[1]), h23 = pack_bf16x2(p[2], p[3]);
            const uint32_t l01 = pack_bf16x2(p[0] - bf16_lo(h01), p[1] - bf16_hi(h01));
            const uint32_t l23 = pack_bf16x2(p[2] - bf16_lo(h23), p[3] - bf16_hi(h23));
            pb[j] = as_bf16x8(u32x4{h01, h23, l01, l23});
        }
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
                const u32x2 va = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)(vt + vposj(mb, j))));
                oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(u32x4{va[0], va[1], va[0], va[1]}),
                                                                   pb[j], oacc[mb], 0, 0, 0);
            }
    }

    // Lane (n, h) of M block mb holds value dims 32 mb + 8 jj + 4 h + 0..3 (jj = 0..3) of row n.
    if (!row_ok) return;
    const int64_t row = (int64_t(b) * a.q_len + t) * a.Hq + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    const float lse2 = l_run > 0.f ? m_run + __log2f(l_run) : kNegInf;
    if (DIRECT) {
        uint16_t *o = a.out + row * kD + 4 * h;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *reinterpret_cast<uint2 *>(o + 32 * mb + 8 * jj) =
                    make_uint2(pack_bf16x2(oacc[mb][4 * jj] * inv, oacc[mb][4 * jj + 1] * inv),
                               pack_bf16x2(oacc[mb][4 * jj + 2] * inv, oacc[mb][4 * jj + 3] * inv));
        if (h == 0 && a.lse2_out) a.lse2_out[row] = lse2;
    } else {
        const int64_t prow = a.part_start ? (int64_t(rest) * a.q_len + t) * a.Hq + head
                                          : row * a.np + part;
        float *o = a.part_o + prow * kD + 4 * h;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                store_partial(reinterpret_cast<f32x4 *>(o + 32 * mb + 8 * jj),
                              f32x4{oacc[mb][4 * jj] * inv, oacc[mb][4 * jj + 1] * inv,
                                    oacc[mb][4 * jj + 2] * inv, oacc[mb][4 * jj + 3] * inv});
        if (h == 0) a.part_lse2[prow] = lse2;
    }
}

hipError_t launch_rows32(const GqaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(a.total_ctas), block(64 * kWaves32);
    if (direct)
        hipLaunchKernelGGL((gqa_rows32_kernel<true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gqa_rows32_kernel<false>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int W>
hipError_t launch_rows(const GqaSplitArgs &a, bool direct, hipStream_t s) {
    const dim3 grid(a.total_ctas), block(64 * W);
    if (direct)
        hipLaunchKernelGGL((gqa_split_kernel<true, W>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((gqa_split_kernel<false, W>), grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace

int gqa_heads_per_cta(int num_kv_heads, int rows_per_group) {
    return num_kv_heads % 2 == 0 && rows_per_group <= 16 ? 2 : 0;
}

hipError_t launch_gqa_split(const GqaSplitArgs &a, bool direct, hipStream_t s) {
    if (a.block_k % kTile) return hipErrorInvalidValue;
    const int rows = a.q_len * a.group;
    if (gqa_heads_per_cta(a.Hkv, rows) == 2) return launch_pair(a, direct, s);
    if (rows <= 16) return launch_rows<1>(a, direct, s);
    if (rows <= 32) return launch_rows<2>(a, direct, s);
    if (a.block_k % kTile32) return hipErrorInvalidValue;
    if (rows <= 64) return launch_rows32(a, direct, s);
    return hipErrorInvalidValue;
}

}  // namespace gqa
