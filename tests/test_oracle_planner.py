"""Pins of the oracle planner and tile rule against what the pages fix (CPU only).

Planner: Modular MAX API page "hip_mha_decoding_num_partitions".  Tile rule: AITER issue
"[Perf] pa_decode_sparse: BLOCK_K=64 is suboptimal above the CU count"."""
import itertools

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
