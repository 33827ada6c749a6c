"""The C-ABI library on the host (no GPU): exports, planner parity with the oracle, and the
argument checks that run before anything is enqueued."""
import ctypes
import itertools
import os
import re
import subprocess

import pytest

import gqa_plan_splits_amd as g
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced by the host checks


def header_functions():
    text = open(os.path.join(ROOT, "include", "gqa_splits.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^(?:int|const char \*)\s*\*?(\w+)\(", text, flags=re.M))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("plan_splits", "block_k_for", "decode_split", "splitk_reduce",
                     "decode_workspace_bytes", "decode", "status_string"):
        assert required in names


def test_library_exports_every_declared_symbol():
    names = header_functions()
    out = subprocess.run(["nm", "-D", "--defined-only", g.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = names - exported
    assert not missing, missing
    assert set(g.exported_symbols()) == names


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5):
        assert g.status_string(code) != "unknown status"
    assert g.status_string(-99) == "unknown status"


@pytest.mark.parametrize("is_mla", [False, True])
def test_planner_matches_oracle_dense_sweep(is_mla):
    bss = [1, 2, 3, 4, 5, 7, 8, 9, 16, 17, 24, 32, 34, 64, 100, 128, 256, 512]
    nks = [0, 1, 127, 128, 255, 256, 257, 1000, 1280, 1281, 2048, 4096, 8191, 32768, 65280,
           65281, 65536, 81920, 131072, 150000, 262144, 1 << 20]
    hpgs = [1, 2, 4, 8, 12, 16, 24, 32, 48, 64, 96, 128, 256]
    sms = [1, 32, 80, 256, 260, 304]
    for bs, nk, hpg, sm in itertools.product(bss, nks, hpgs, sms):
        assert g.plan_splits(bs, nk, hpg, sm, is_mla) == oracle.plan_splits(bs, nk, hpg, sm, is_mla), \
            (bs, nk, hpg, sm, is_mla)


def test_block_k_matches_oracle():
    for ctas, sm in itertools.product([1, 2, 100, 255, 256, 257, 512, 8192], [1, 80, 256, 304]):
        assert g.block_k_for(ctas, sm) == oracle.block_k(ctas, sm)


def test_sparse_planner_matches_oracle_sweep():
    # bit-exact against the oracle's reading of the FlashInfer sparse planner page
    tokens = [1, 2, 3, 4, 7, 8, 16, 24, 32, 34, 48, 60, 64, 100, 128, 170, 200, 250, 256, 512, 1024]
    heads = [1, 16, 17, 32, 64, 128]
    topks = [0, 64, 65, 128, 129, 256, 512, 1000, 1024, 1025, 2048, 4096]
    extras = [0, 64, 100, 512]
    for nt, nh, topk, extra in itertools.product(tokens, heads, topks, extras):
        for sms, mx, ht in ((48, 16, 1), (170, 16, 1), (188, 16, 2), (256, 16, 4), (256, 4, 4), (304, 64, 1)):
            want = oracle.plan_sparse_splits(nt, nh, topk, extra, num_sms=sms, max_splits=mx, head_tiles=ht)
            if want is None:
                with pytest.raises(g.GqaError):
                    g.plan_sparse_splits(nt, nh, topk, extra, num_sms=sms, max_splits=mx, head_tiles=ht)
            else:
                assert g.plan_sparse_splits(nt, nh, topk, extra, num_sms=sms, max_splits=mx,
                                            head_tiles=ht) == want, (nt, nh, topk, extra, sms, mx, ht)


def test_sparse_planner_rejections():
    for args in [(0, 64, 2048), (1, 0, 2048), (1, 64, -1)]:
        with pytest.raises(g.GqaError):
            g.plan_sparse_splits(*args, num_sms=256)
    with pytest.raises(g.GqaError):
        g.plan_sparse_splits(1, 64, 2048, -1, num_sms=256)
    with pytest.raises(g.GqaError):
        g.plan_sparse_splits(1, 64, 2048, num_sms=256, max_splits=0)
    with pytest.raises(g.GqaError):
        g.plan_sparse_splits(1, 64, 2048, num_sms=256, head_tiles=0)
    with pytest.raises(g.GqaError):   # 32 chunks need 2 splits
        g.plan_sparse_splits(1, 64, 2048, num_sms=256, max_splits=1)


def test_sparse_measured_rule_properties():
    # the MI355X-measured variant: a power of two within max_splits whose grid stays within one
    # wave of CUs and leaves two chunks per CTA (one for a lone CTA); two chunks never split
    for nt, nh, topk, extra, sm, mx in itertools.product([1, 2, 3, 8, 24, 64, 256, 300], [16, 64, 128],
                                                         [0, 64, 128, 192, 1024, 2048, 4096], [0, 256],
                                                         [80, 256], [1, 16, 32, 256]):
        ns = g.plan_sparse_splits_measured(nt, nh, topk, extra, sm_count=sm, max_splits=mx)
        chunks = -(-topk // 64) + -(-extra // 64)
        ctas = nt * -(-nh // 64)
        assert ns >= 1 and ns & (ns - 1) == 0 and ns <= mx
        if chunks <= 2:
            assert ns == 1
        elif ns > 1:
            assert ctas * ns <= sm
            assert chunks >= (ns if ctas == 1 else 2 * ns)
            # and the next power of two breaks one of the bounds
            n2 = 2 * ns
            assert n2 > mx or ctas * n2 > sm or chunks < (n2 if ctas == 1 else 2 * n2)
    with pytest.raises(g.GqaError):
        g.plan_sparse_splits_measured(0, 64, 2048, sm_count=256)


def test_planner_rejections():
    for args in [(0, 1, 1, 256), (1, -1, 1, 256), (1, 1, 0, 256)]:
        with pytest.raises(g.GqaError) as e:
            g.plan_splits(*args, is_mla=True)
        assert e.value.status == -1
    with pytest.raises(g.GqaError):
        g.block_k_for(0, 256)
    with pytest.raises(g.GqaError):
        g.block_k_for(10, 0)


def mla_fake(B=2, q_len=1, H=64, d_qk=576, d_v=512, max_keys=65536):
    p = g.DecodeProblem()
    p.kind, p.fp8_format = g.KIND_MLA_FUSED, g.FP8_E4M3FN
    p.batch, p.q_len, p.num_heads, p.num_kv_heads = B, q_len, H, 1
    p.d_qk, p.d_rope, p.d_v, p.page_size, p.max_num_keys = d_qk, 64, d_v, 1, max_keys
    p.q, p.q_stride_tok, p.q_stride_head = FAKE, H * (d_qk - 64), d_qk - 64
    p.q_pe, p.q_pe_stride_tok, p.q_pe_stride_head = FAKE, H * 64, 64
    p.kv, p.kv_stride_row = FAKE, d_qk
    p.kv_indices = p.kv_indptr = p.seq_lens = FAKE
    p.scale, p.kv_scale = d_qk ** -0.5, 1 / 32
    return p


def gqa_fake(B=32, Hq=64, Hkv=8, page=16, q_len=1, max_keys=32768):
    p = g.DecodeProblem()
    p.kind = g.KIND_GQA_PAGED
    p.batch, p.q_len, p.num_heads, p.num_kv_heads = B, q_len, Hq, Hkv
    p.d_qk, p.d_rope, p.d_v, p.page_size, p.max_num_keys = 128, 0, 128, page, max_keys
    p.q, p.q_stride_tok, p.q_stride_head = FAKE, Hq * 128, 128
    p.k_cache = p.v_cache = FAKE
    p.kv_indices = p.kv_indptr = p.seq_lens = FAKE
    p.scale, p.kv_scale = 128 ** -0.5, 1.0
    return p


@pytest.mark.parametrize("B,q_len,H,keys", [(1, 1, 16, 4096), (2, 1, 64, 65536), (8, 1, 64, 131072),
                                            (16, 1, 64, 131072), (8, 4, 64, 131072),
                                            (16, 4, 64, 131072), (24, 1, 64, 2048),
                                            (34, 1, 64, 2048), (256, 1, 64, 2048)])
def test_decode_plan_mla_matches_oracle(B, q_len, H, keys):
    p = mla_fake(B=B, q_len=q_len, H=H, max_keys=keys)
    np_, bk = g.decode_plan(p, 0, 0, 256)
    # the planner sees the query rows packed per request; the tile rule sees the CTAs the split
    # launches (64 query rows each)
    want_np = oracle.plan_splits(B, keys, q_len * H, 256, True)
    assert np_ == want_np
    assert bk == oracle.block_k(B * want_np * -(-(q_len * H) // 64), 256)


def test_decode_plan_gqa_matches_oracle():
    p = gqa_fake()
    np_, bk = g.decode_plan(p, 0, 0, 256)
    assert np_ == oracle.plan_splits(32, 32768, 8, 256, False)
    assert bk == oracle.block_k(32 * np_ * 8, 256)
    assert (np_, bk) == (32, 32)


def test_decode_plan_explicit_overrides():
    p = mla_fake()
    assert g.decode_plan(p, 4, 32, 256) == (4, 32)
    assert g.decode_plan(p, 1, 64, 256) == (1, 64)


def expect_status(fn, status):
    with pytest.raises(g.GqaError) as e:
        fn()
    assert e.value.status == status, (e.value.status, status)


@pytest.mark.parametrize("field,value,status", [
    ("batch", 0, -1), ("q_len", 0, -1), ("num_heads", 0, -1), ("max_num_keys", -1, -1),
    ("num_heads", 129, -2), ("q", 0, -1), ("kv", 0, -1), ("q_pe", 0, -1), ("kv_indices", 0, -1),
    ("kv_indptr", 0, -1), ("seq_lens", 0, -1), ("num_kv_heads", 2, -1), ("kind", 7, -1),
    ("fp8_format", 1, -2), ("fp8_format", 5, -1), ("d_qk", 128, -2), ("d_v", 256, -2),
    ("page_size", 16, -2), ("kv_stride_row", 500, -2), ("kv_stride_row", 1 << 32, -2), ("q", FAKE + 8, -2),
    ("q_stride_head", 4, -2), ("scale", 0.0, -1), ("kv_scale", 0.0, -1),
])
def test_mla_rejections(field, value, status):
    p = mla_fake()
    setattr(p, field, value)
    expect_status(lambda: g.decode_plan(p, 4, 32, 256), status)
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), status)
    expect_status(lambda: g.decode(p, FAKE, np=4, block_k=32, workspace=None), status)


@pytest.mark.parametrize("field,value,status", [
    ("num_kv_heads", 0, -1), ("num_kv_heads", 7, -1), ("k_cache", 0, -1), ("v_cache", 0, -1),
    ("d_qk", 64, -2), ("d_rope", 64, -2), ("page_size", 12, -2), ("page_size", 4, -2),
    ("q_len", 9, -2),  # 9 x 8 = 72 query rows per kv head: above the four 16-row blocks
])
def test_gqa_rejections(field, value, status):
    p = gqa_fake()
    setattr(p, field, value)
    expect_status(lambda: g.decode_plan(p, 4, 32, 256), status)
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), status)


@pytest.mark.parametrize("Hq,Hkv,q_len", [(64, 1, 1), (32, 1, 2), (16, 1, 4), (64, 8, 8), (24, 1, 1)])
def test_gqa_row_blocks_accepted(Hq, Hkv, q_len):
    # up to 64 query rows per kv head (four blocks of 16) plan like any other GQA problem
    p = gqa_fake(Hq=Hq, Hkv=Hkv, q_len=q_len)
    np_, bk = g.decode_plan(p, 0, 0, 256)
    assert np_ == oracle.plan_splits(32, 32768, Hkv, 256, False)
    assert bk == oracle.block_k(32 * np_ * Hkv, 256)


def test_split_argument_rejections():
    p = mla_fake()
    expect_status(lambda: g.decode_split(p, 0, 32, FAKE, FAKE), -2)
    expect_status(lambda: g.decode_split(p, 257, 32, FAKE, FAKE), -2)
    expect_status(lambda: g.decode_split(p, 4, 48, FAKE, FAKE), -2)
    expect_status(lambda: g.decode_split(p, 4, 32, 0, FAKE), -1)
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, 0), -1)


def test_reduce_argument_rejections():
    expect_status(lambda: g.splitk_reduce(-1, 4, 512, FAKE, FAKE, FAKE), -1)
    expect_status(lambda: g.splitk_reduce(8, 0, 512, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.splitk_reduce(8, 257, 512, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.splitk_reduce(8, 4, 510, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.splitk_reduce(8, 4, 512, 0, FAKE, FAKE), -1)
    expect_status(lambda: g.splitk_reduce(8, 4, 512, FAKE, FAKE, 0), -1)
    g.splitk_reduce(0, 4, 512, FAKE, FAKE, FAKE)   # no rows: nothing to enqueue


def test_context_parallel_rejections():
    # rank outside the world, a world without global lengths, shapes that have no DCP kernel
    p = mla_fake()
    p.glen, p.cp_world, p.cp_rank = FAKE, 4, 4
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p.cp_rank = -1
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p = mla_fake()
    p.cp_world, p.cp_rank = 4, 1
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p = mla_fake()
    p.cp_rank = 1   # a rank without a world
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p = mla_fake()
    p.glen, p.cp_world, p.cp_rank = FAKE, 257, 0
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = mla_fake()
    p.d_qk, p.d_v = 512, 448   # sparse rows
    p.glen, p.cp_world, p.cp_rank = FAKE, 2, 1
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = gqa_fake()
    p.glen, p.cp_world, p.cp_rank = FAKE, 2, 1
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)


def test_second_cache_rejections():
    # a second cache needs its index lists, sparse rows, q_len 1, no context parallelism and the
    # pool's row stride
    def sparse():
        p = mla_fake(d_qk=512, d_v=448, max_keys=4096)
        p.kv2, p.kv2_indices, p.kv2_indptr = FAKE, FAKE, FAKE
        return p
    assert g.decode_workspace_bytes(sparse(), 4) > 0
    p = sparse()
    p.kv2_indices = None
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p = sparse()
    p.kv2 = None
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)
    p = sparse()
    p.q_len = 2
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = mla_fake()   # wide rows
    p.kv2, p.kv2_indices, p.kv2_indptr = FAKE, FAKE, FAKE
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = sparse()
    p.kv2_stride_row = 1024   # not the pool's stride
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = sparse()
    p.glen, p.cp_world, p.cp_rank = FAKE, 2, 0
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = gqa_fake()
    p.kv2, p.kv2_indices, p.kv2_indptr = FAKE, FAKE, FAKE
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)


def test_bf16_pool_checks():
    # a bf16 pool: rows of 2 bytes per element (stride >= 2 d_qk); a second cache at its stride
    p = mla_fake()
    p.fp8_format = g.KV_BF16
    p.kv_stride_row = 576
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p.kv_stride_row = 1152
    assert g.decode_plan(p, 4, 32, 256) == (4, 32)
    p = mla_fake(d_qk=512, d_v=448, max_keys=4096)
    p.fp8_format, p.kv_stride_row = g.KV_BF16, 1024
    assert g.decode_plan(p, 0, 0, 256)[0] >= 1
    p.kv2, p.kv2_indices, p.kv2_indptr = FAKE, FAKE, FAKE   # a second bf16 cache
    assert g.decode_workspace_bytes(p, 4) > 0
    p.kv2_stride_row = 512   # not the pool's stride
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -2)
    p = mla_fake()
    p.fp8_format = 3
    expect_status(lambda: g.decode_split(p, 4, 32, FAKE, FAKE), -1)


def test_proportional_plan_argument_rejections():
    def plan(seq=FAKE, batch=4, budget=16, cap=8, bk=32, start=FAKE, chunk=FAKE):
        return lambda: g.plan_proportional_device(seq, None, batch, budget, cap, bk, start, chunk)
    expect_status(plan(seq=None), -1)
    expect_status(plan(start=None), -1)
    expect_status(plan(chunk=None), -1)
    expect_status(plan(batch=0), -1)
    expect_status(plan(budget=0), -1)
    expect_status(plan(cap=0), -1)
    expect_status(plan(cap=257), -2)
    expect_status(plan(bk=16), -2)
    expect_status(plan(budget=(1 << 30) + 1), -2)


def test_decode_proportional_layout_and_rejections():
    lib = g._lib._load()

    def call(p, np_, cap, ws_bytes, out=FAKE, ws=0x100000):
        return lib.decode_proportional(ctypes.byref(p), np_, cap, 32, ws, ws_bytes, out, None, None)

    # workspace: slot-major partials of batch * np slots (decode's bytes for np), then the two
    # plan tables, each 256-byte aligned; cap does not change it
    p = mla_fake(B=3, H=64)
    rows, dv = 3 * 64, 512
    want = rows * 8 * dv * 4 + rows * 8 * 4 + 256 + 256
    assert g.decode_proportional_workspace_bytes(p, 8) == want
    assert g.decode_proportional_workspace_bytes(p, 8, 5) == want
    assert g.decode_proportional_workspace_bytes(p, 8) == g.decode_workspace_bytes(p, 8) + 512
    assert call(p, 8, 0, want - 1) == -3
    assert call(p, 8, 0, want, out=None) == -1
    assert call(p, 8, 0, want, ws=0x100010) == -1     # workspace not 256-byte aligned
    assert call(p, 8, 257, 1 << 40) == -2
    assert call(p, 257, 0, 1 << 40) == -2
    p.glen, p.cp_world, p.cp_rank = FAKE, 2, 0
    assert call(p, 8, 0, 1 << 40) == -2
    assert call(p, 8, 0, want, out=FAKE + 4) == -2   # output not 8-byte aligned
    q = gqa_fake(B=5)
    rows = 5 * 64
    assert g.decode_proportional_workspace_bytes(q, 3) == rows * 3 * 128 * 4 + 3840 + 512


def test_merge_ranks_argument_rejections():
    expect_status(lambda: g.merge_ranks(4, -1, 512, FAKE, FAKE, FAKE), -1)
    expect_status(lambda: g.merge_ranks(0, 8, 512, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.merge_ranks(257, 8, 512, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.merge_ranks(4, 8, 510, FAKE, FAKE, FAKE), -2)
    expect_status(lambda: g.merge_ranks(4, 8, 512, FAKE + 4, FAKE, FAKE), -2)
    expect_status(lambda: g.merge_ranks(4, 8, 512, 0, FAKE, FAKE), -1)
    expect_status(lambda: g.merge_ranks(4, 8, 512, FAKE, 0, FAKE), -1)
    expect_status(lambda: g.merge_ranks(4, 8, 512, FAKE, FAKE, 0), -1)
    g.merge_ranks(4, 0, 512, FAKE, FAKE, FAKE)   # no rows: nothing to enqueue


def test_workspace_contract():
    p = mla_fake(B=2, H=64)
    need = g.decode_workspace_bytes(p, 64)
    rows = 2 * 64
    assert need >= rows * 64 * 512 * 4 + rows * 64 * 4
    assert need % 256 == 0
    assert g.decode_workspace_bytes(p, 1) == 0
    lib = g._lib._load()
    rc = lib.decode(ctypes.byref(p), 64, 64, ctypes.c_void_p(FAKE), need - 256,
                    ctypes.c_void_p(FAKE), None, None)
    assert rc == -3
    rc = lib.decode(ctypes.byref(p), 64, 64, None, need, ctypes.c_void_p(FAKE), None, None)
    assert rc == -1


@pytest.mark.parametrize("B,S,hkv,best", [(8, 32768, 1, 128), (64, 8192, 1, 16), (8, 32768, 8, 16),
                                          (64, 8192, 8, 8), (32, 32768, 8, 32)])
def test_gqa_measured_planner_hits_the_measured_best(B, S, hkv, best):
    # the best partition counts the planner-branch sweep measured on MI355X (256 CUs); at
    # 8 x 32768 with 8 kv heads np 16 and 64 measured within 0.1 % of each other
    assert g.plan_gqa_splits_measured(B, S, hkv, 256) == best


def test_gqa_measured_planner_properties():
    for B in (1, 2, 3, 8, 31, 64, 200):
        for S in (0, 100, 256, 1000, 8192, 65536, 1 << 20):
            for hkv in (1, 2, 8, 16):
                for sm in (80, 256):
                    base = g.plan_splits(B, S, hkv, sm, False)
                    n = g.plan_gqa_splits_measured(B, S, hkv, sm)
                    assert base <= n <= 256
                    if n > base:
                        assert n & (n - 1) == 0 and n * 256 <= S
                        # the smallest such power of two: half of it leaves the chip short
                        assert n == 1 or B * hkv * (n // 2) < 4 * sm
    expect_status(lambda: g.plan_gqa_splits_measured(0, 100, 1, 256), -1)
    expect_status(lambda: g.plan_gqa_splits_measured(1, -1, 1, 256), -1)
    expect_status(lambda: g.plan_gqa_splits_measured(1, 100, 0, 256), -1)


def test_decode_scratch_rejects_partials_beyond_the_static_array():
    # checked on the host before anything touches the device: 4096 rows x 256 partitions of
    # 512 fp32 values need 2 GiB, beyond GQA_SCRATCH_BYTES
    prob = g.DecodeProblem()
    prob.kind, prob.fp8_format = g.KIND_MLA_FUSED, g.FP8_E4M3FN
    prob.batch, prob.q_len, prob.num_heads, prob.num_kv_heads = 64, 1, 64, 1
    prob.d_qk, prob.d_rope, prob.d_v, prob.page_size, prob.max_num_keys = 576, 64, 512, 1, 300
    prob.q = prob.q_pe = prob.kv = prob.kv_indices = prob.kv_indptr = prob.seq_lens = FAKE
    prob.q_stride_tok, prob.q_stride_head = 64 * 512, 512
    prob.q_pe_stride_tok, prob.q_pe_stride_head = 64 * 64, 64
    prob.kv_stride_row = 576
    prob.scale, prob.kv_scale = 576 ** -0.5, 1 / 32
    assert g.decode_workspace_bytes(prob, 256) > g.SCRATCH_BYTES
    with pytest.raises(g.GqaError) as e:
        g.decode_scratch(prob, FAKE, FAKE, np=256, block_k=32)
    assert e.value.status == -3 and "static scratch holds" in str(e.value)
    # a plan that fits goes past this check (and would need the device)
    assert g.decode_workspace_bytes(prob, 2) <= g.SCRATCH_BYTES


def test_mla_measured_planner_properties():
    for B in (1, 2, 3, 8, 16, 64, 300):
        for S in (0, 100, 255, 256, 4096, 16384, 131072, 1 << 20):
            for rows in (1, 16, 64, 65, 128, 256):
                for sm in (80, 256):
                    n = g.plan_mla_splits_measured(B, S, rows, sm)
                    ctas = B * -(-rows // 64)
                    assert 1 <= n <= 256 and n & (n - 1) == 0
                    if n > 1:
                        assert ctas * n <= sm and n * 256 <= S
                    # the largest such power of two
                    assert 2 * n > 256 or ctas * 2 * n > sm or 2 * n * 256 > S
    # the two-wave exception of the pages' planner (MLA, 16 heads) becomes one wave of CTAs
    assert g.plan_splits(4, 65536, 16, 256, True) == 128
    assert g.plan_mla_splits_measured(4, 65536, 16, 256) == 64
    expect_status(lambda: g.plan_mla_splits_measured(0, 100, 64, 256), -1)
    expect_status(lambda: g.plan_mla_splits_measured(1, -1, 64, 256), -1)
    expect_status(lambda: g.plan_mla_splits_measured(1, 100, 0, 256), -1)


def test_ceiling_argument_rejections():
    expect_status(lambda: g.bw_stream_read(FAKE, 4096 * 3, 2), -2)      # not a multiple of ctas * 4 KiB
    expect_status(lambda: g.bw_stream_read(FAKE + 4, 4096, 1), -2)      # misaligned
    expect_status(lambda: g.bw_stream_read(FAKE, 4096, 0), -1)
    expect_status(lambda: g.bw_gather_rows(FAKE, 300, FAKE, 64, 1), -2)  # row width
    expect_status(lambda: g.bw_gather_rows(FAKE, 576, FAKE, 65, 1), -2)  # not 64-row groups
    expect_status(lambda: g.bw_gather_rows(FAKE, 576, FAKE, -64, 1), -1)
    expect_status(lambda: g.bw_gather_whole_rows(FAKE, 300, FAKE, 64, 1), -2)
    expect_status(lambda: g.bw_gather_whole_rows(FAKE, 576, FAKE, 65, 1), -2)
    expect_status(lambda: g.bw_gather_whole_rows(FAKE, 576, FAKE, -64, 1), -1)


@pytest.mark.parametrize("B,S,rows,best", [(4, 65536, 16, 64), (16, 16384, 16, 16), (2, 65536, 64, 128),
                                           (4, 65536, 32, 64), (16, 16384, 32, 16), (4, 65536, 128, 32),
                                           (16, 16384, 128, 8), (16, 131072, 64, 16), (8, 131072, 64, 32)])
def test_mla_measured_planner_hits_the_measured_best(B, S, rows, best):
    # the best partition counts of the planner-branch sweep on MI355X (256 CUs), graph-replayed
    # decode calls at every power-of-two np; the last two rows are the long-context workloads
    assert g.plan_mla_splits_measured(B, S, rows, 256) == best
