"""Pins of the oracle planner and tile rule against what the pages fix (CPU only).

Planner: Modular MAX API page "hip_mha_decoding_num_partitions".  Tile rule: AITER issue
"[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the CU count"."""
import itertools

import numpy as np

import pytest

import oracle


@pytest.mark.parametrize("row", range(7))
def test_phase0_sweep_table(golden, row):
    bs, nk, hpg, sm, is_mla, expected = golden("planner_phase0_sweep.txt")[row]
    assert oracle.plan_splits(bs, nk, hpg, sm, bool(is_mla)) == expected


def test_page_statements(golden):
    for bs, nk, hpg, sm, is_mla, expected in golden("planner_statements.txt"):
        assert oracle.plan_splits(bs, nk, hpg, sm, bool(is_mla)) == expected, (bs, nk, hpg)


def test_only_64k_reaches_256_at_bs1_h16():
    # Reducer-constraint paragraph: 256 partitions are reached only from 64K keys (256 pages of
    # 256 keys) up; below that the page count limits the partition count.
    for nk in list(range(0, 70000, 97)) + [65280, 65281, 65536]:
        np_ = oracle.plan_splits(1, nk, 16, 256, True)
        pages = -(-nk // 256)
        if pages >= 256:
            assert np_ == 256
        else:
            assert np_ == max(1, pages)


def test_reducer_cap_and_mha_caps():
    # Tunables list and MHA bullet: MLA-style is capped at the reducer's 256 partitions, the
    # MHA-style branch at 64, and at 32 when there are exactly 16 kv heads and batch >= 8.
    for bs, nk, hpg, sm in itertools.product([1, 2, 3, 8, 16, 64], [0, 1, 300, 5000, 65536, 1 << 20],
                                             [1, 2, 4, 8, 16, 24, 32, 64, 128], [32, 80, 256, 304]):
        for is_mla in (False, True):
            np_ = oracle.plan_splits(bs, nk, hpg, sm, is_mla)
            pages = -(-nk // (128 if (not is_mla and hpg == 1) else 256))
            assert 1 <= np_ <= max(1, pages)
            if is_mla or hpg >= 32:
                assert np_ <= 256
            else:
                assert np_ <= 64
                if hpg == 16 and bs >= 8:
                    assert np_ <= 32


def test_bucket_is_power_of_two_unless_page_limited():
    # Phase-0 sweep: a work floor of 103 is rounded up to 128, so targets are bucketed to powers
    # of two; only the page floor (never more partitions than 256-key pages) can leave another
    # value.
    for bs, nk, hpg in itertools.product([1, 2, 4, 8, 16, 32], [1000, 4096, 50000, 131072, 400000],
                                         [16, 32, 64, 128]):
        np_ = oracle.plan_splits(bs, nk, hpg, 256, True)
        pages = -(-nk // 256)
        assert (np_ & (np_ - 1)) == 0 or np_ == pages


def test_single_kv_head_mha_uses_finer_pages():
    # EXCEPTION paragraph: single-kv-head MHA changes under the two-wave rule because its split
    # pages are 128 keys instead of 256, doubling the page count.  8192 keys are
    # 64 pages of 128 keys; batch 16 with one kv head is 16 CTAs per partition, so the two-wave
    # target 2*256 // 16 = 32 applies, where the one-wave clamp of work_floor 13 would give 16.
    assert oracle.plan_splits(16, 8192, 1, 256, False) == 32
    # two kv heads: 256-key pages (32 of them), 32 CTAs, clamp(7, 8, 16) = 8
    assert oracle.plan_splits(16, 8192, 2, 256, False) == 8
    # and the MHA-style branch stays pinned <= 64 even when two waves would ask for more
    assert oracle.plan_splits(4, 32768, 1, 256, False) == 64


def test_invalid_arguments():
    assert oracle.plan_splits(0, 10, 64, 256, True) == -1
    assert oracle.plan_splits(1, -1, 64, 256, True) == -1
    assert oracle.plan_splits(1, 10, 0, 256, True) == -1
    assert oracle.plan_splits(1, 10, 64, 0, True) == -1
    assert oracle.block_k(0, 256) == -1
    assert oracle.block_k(10, 0) == -1


def test_block_k_rule():
    # Tile rule: 32 when the launch has more CTAs than the device has CUs, else 64 (strict).
    assert oracle.block_k(1, 256) == 64
    assert oracle.block_k(256, 256) == 64
    assert oracle.block_k(257, 256) == 32
    assert oracle.block_k(8192, 256) == 32


def test_block_k_tracks_ctas_not_queries():
    # The issue keys the choice on CTAs (queries x splits x head blocks), not on the query count,
    # which is why it is not monotonic in queries: 32 queries can launch fewer CTAs than 34.  With
    # this planner
    # (64 heads -> 2 head blocks of 32, 2048 keys per query) 32 queries give 256 CTAs and 34
    # give 272.
    def ctas(nq):
        return nq * oracle.plan_splits(nq, 2048, 64, 256, True) * 2
    assert ctas(32) == 256 and oracle.block_k(ctas(32), 256) == 64
    assert ctas(34) == 272 and oracle.block_k(ctas(34), 256) == 32
    assert ctas(24) > 256 and oracle.block_k(ctas(24), 256) == 32


def test_two_wave_is_read_left_to_right():
    # Reading, not a page value: the page writes the two-wave bound as 2 x sm_count // ctas with
    # no parentheses; it is evaluated left to right, (2 * sm) // ctas.  The worked table cannot
    # tell the readings apart (its CTA counts all divide 256).  At sm=260 and 8 CTAs the two
    # readings give 65 and 64, which bucket to 128 and 64.
    assert oracle.plan_splits(4, 1 << 20, 64, 260, True) == 128


# ---- sparse top-k planner: FlashInfer API page "cake_sparse_mla_sm120_dsv4_nvfp4_plan_splits"

def test_sparse_planner_page_statements(golden):
    for nt, nh, topk, extra, sms, mx, ht, ns, cpb in golden("sparse_planner_statements.txt"):
        got = oracle.plan_sparse_splits(nt, nh, topk, extra, num_sms=sms, max_splits=mx, head_tiles=ht)
        assert got == (ns, cpb), (nt, nh, topk, extra, sms, mx, ht, got)


def test_sparse_planner_index_table_bound():
    # "chunks_per_block <= max_chunks_per_block always holds": more than 1024 candidates force at
    # least ceil(chunks / 16) splits, and a max_splits below that is an error.
    for topk in (0, 64, 1000, 1024, 1025, 2048, 4096, 8192):
        chunks = -(-topk // 64)
        forced = max(1, -(-chunks // 16))
        for mx in (1, 2, 4, 8, 16, 64):
            for nt, sms in ((1, 48), (3, 170), (200, 170), (1, 256), (512, 256)):
                got = oracle.plan_sparse_splits(nt, 16, topk, 0, num_sms=sms, max_splits=mx)
                if forced > mx:
                    assert got is None
                    continue
                ns, cpb = got
                assert forced <= ns <= mx
                assert cpb <= 16 and ns * cpb >= chunks
                if chunks <= 2:
                    assert ns == 1


def test_sparse_planner_split_is_largest_admissible():
    # The small-grid rule, re-checked by brute force over every power of two: the planner's split
    # is the largest one that keeps the grid within 80 % of the SMs (SMs / 3 and gather streams
    # within SMs / 6 below 64 SMs) and leaves two chunks per CTA (one for a lone CTA on a large
    # device), unless the index table forces more.
    for sms in (48, 170, 188, 256):
        for nt in (1, 2, 3, 5, 8, 16):
            for nh in (16, 64, 128):
                for topk in (192, 256, 512, 1024):
                    grid = nt * -(-nh // 16)
                    if 10 * grid > 4 * sms:
                        continue
                    chunks = -(-topk // 64)
                    ns, _ = oracle.plan_sparse_splits(nt, nh, topk, 0, num_sms=sms)
                    lone = grid == 1 and sms >= 64
                    best = 1
                    for s in (1, 2, 4, 8, 16):
                        room = (grid * s <= sms // 3 and nt * s <= sms // 6) if sms < 64 else 10 * grid * s <= 8 * sms
                        enough = chunks >= s if lone else chunks >= 2 * s
                        if room and enough and chunks > 2:
                            best = s
                    assert ns == best, (sms, nt, nh, topk, ns, best)


# ---------------------------------------------------------------------------------------------
# Length-proportional partitions (moonmath-amd README, "VarlenPlan": planning on the GPU from
# device-side lengths; the proportional rule is this library's reading)
# ---------------------------------------------------------------------------------------------

def test_proportional_plan_worked_example():
    # lengths 1000, 0, 31, 5000 over 8 partitions, at most 4 per request, 32-key tiles, by hand.
    # 5000 keys need more than 4 partitions below 1250 keys each, so they take 4 of 1280 keys
    # whatever the common length c; 31 keys take 1 and 0 keys none.  1000 keys take 4 partitions
    # for c < 334 (capped at 4 of 256 below 250) -- 9 in all, over the budget -- and 3 for
    # 334 <= c < 500, 8 in all.  The smallest multiple of 32 from 334 on is 352.
    start, chunk = oracle.proportional_plan([1000, 0, 31, 5000], budget=8, cap=4, block_k=32)
    assert start == [0, 3, 3, 4, 8]
    assert chunk == [352, 352, 352, 1280]


def _check_plan(lengths, budget, cap, bk):
    start, chunk = oracle.proportional_plan(lengths, budget, cap, bk)
    B = len(lengths)
    assert len(start) == B + 1 and start[0] == 0

    def count(c):   # partitions of the batch under common length c, by the rule's definition
        n = 0
        for L in lengths:
            k = -(-L // c)
            if k > cap:
                cb = bk
                while -(-L // cb) > cap:   # brute force: smallest bk multiple within cap
                    cb += bk
                k = -(-L // cb)
            n += k
        return n

    common = [chunk[b] for b in range(B) if -(-lengths[b] // chunk[b]) <= cap or lengths[b] == 0]
    nonempty = sum(1 for L in lengths if L > 0)
    for b, L in enumerate(lengths):
        k = start[b + 1] - start[b]
        assert chunk[b] % bk == 0 and chunk[b] >= bk
        assert 0 <= k <= cap
        # the partitions cover the request's keys and none of them is empty
        assert k * chunk[b] >= L and (k - 1) * chunk[b] < max(L, 1)
    if budget >= nonempty:
        assert start[-1] <= budget
        # minimality of the common length: one block_k shorter overflows the budget
        c = min(common) if common else None
        if c is not None and c > bk:
            assert count(c - bk) > budget
            assert count(c) == start[-1]


@pytest.mark.parametrize("seed", range(40))
def test_proportional_plan_invariants_random(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 40))
    kind = seed % 4
    if kind == 0:
        lengths = rng.integers(0, 5000, B).tolist()
    elif kind == 1:
        lengths = rng.integers(1024, 32769, B).tolist()
    elif kind == 2:   # one long request among short ones
        lengths = [int(rng.integers(1, 200)) for _ in range(B)]
        lengths[int(rng.integers(B))] = int(rng.integers(50000, 200000))
    else:
        lengths = [0] * B
    budget = int(rng.integers(1, 8 * B + 2))
    cap = int(rng.integers(1, 257))
    bk = (32, 64)[seed % 2]
    _check_plan(lengths, budget, cap, bk)


@pytest.mark.parametrize("S,B,np_,bk", [(65536, 2, 64, 32), (131072, 16, 16, 32), (1000, 3, 7, 64),
                                        (33, 5, 4, 32), (1, 1, 1, 64)])
def test_proportional_plan_uniform_lengths_is_the_equal_split(S, B, np_, bk):
    # equal lengths with a budget of np per request: every request gets the equal split's
    # partition length ceil(S / np) rounded up to bk, and as many partitions as that split fills
    start, chunk = oracle.proportional_plan([S] * B, budget=B * np_, cap=256, block_k=bk)
    eq = -(-(-(-S // np_)) // bk) * bk
    assert chunk == [eq] * B
    assert [start[b + 1] - start[b] for b in range(B)] == [-(-S // eq)] * B


def test_proportional_plan_empty_batch_and_cap_one():
    start, chunk = oracle.proportional_plan([0, 0, 0], budget=5, cap=8, block_k=64)
    assert start == [0, 0, 0, 0] and chunk == [64, 64, 64]
    # cap 1: every non-empty request is one partition covering all its keys, so 3 partitions fit
    # 100 at any common length and the common length is the smallest, 32: 7 keys fit one such
    # partition, 100 and 4096 keys take one partition of 128 and 4096 keys
    start, chunk = oracle.proportional_plan([100, 7, 0, 4096], budget=100, cap=1, block_k=32)
    assert start == [0, 1, 2, 2, 3]
    assert chunk == [128, 32, 32, 4096]
    # a budget below the non-empty requests: each takes one partition of the longest, rounded up
    start, chunk = oracle.proportional_plan([100, 7, 0, 4096], budget=2, cap=8, block_k=32)
    assert start == [0, 1, 2, 2, 3] and chunk == [4096] * 4
