"""GPU parity of the bf16-cache MLA split (the same fused rows stored as bf16, AITER issue
"[Perf] pa_decode_sparse ...", closing paragraph) against the fp64 CPU oracle over the same bf16
values, element by element, with the bars every MLA output meets (max|dO| <= 1e-2,
max|dO| / max|O_ref| <= 1e-2, |d lse2| <= 1e-4 max(1, |lse2|)).

The kernel multiplies the stored bf16 K directly on the bf16 MFMA (exact products, fp32 sums)
and the softmax weights (fp16) by V converted to fp16 (exact within fp16's normal range).  The
cases: ragged requests over several 32-key tiles, draft windows, skipped keys, head counts with
two row blocks, decode context parallelism, wide dynamic range (large queries, rows spanning 20
octaves, large and fp16-subnormal cache values, a dominant key per tile), and the full-size
workloads on sampled rows in the benchmark's launch configuration."""
import numpy as np
import pytest
import torch

import gqa_plan_splits_amd as g
import workloads
from gpu_util import compare, log, mla_problem, oracle_mla, run_decode, sample_rows
from test_gpu_numerics import compare_bf16_output, fp32_result

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.mark.parametrize("d_qk,d_v", [(576, 512), (512, 448)])
@pytest.mark.parametrize("q_len", [1, 4])
@pytest.mark.parametrize("np_,bk", [(1, 32), (3, 64), (8, 32), (0, 0)])
def test_bf16_ragged_all_rows(d_qk, d_v, q_len, np_, bk):
    # several 32-key tiles per partition, ragged tails, a request shorter than the draft window,
    # an empty request, and 40 heads (a partial row block)
    lens = [1000, 37, 2, 0, 2049]
    inp = workloads.mla_inputs(B=5, q_len=q_len, H=40, seq_lens=lens, pool_rows=4000, d_qk=d_qk,
                               d_v=d_v, seed=177, device=DEV, fused_q=(d_qk == 512), kv_dtype="bf16")
    torch.cuda.synchronize()
    log("bf16 ragged d_qk=%d q_len=%d np=%d bk=%d" % (d_qk, q_len, np_, bk))
    out, lse = run_decode(mla_problem(inp), d_v, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "bf16 ragged d_qk=%d q_len=%d np=%d" % (d_qk, q_len, np_))


@pytest.mark.parametrize("np_", [1, 4, 16])
def test_bf16_tiny_all_rows(np_):
    inp = workloads.mla_inputs(B=1, q_len=1, H=16, seq_lens=[4096], pool_rows=4096, seed=7,
                               device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    log("bf16 tiny np=%d" % np_)
    out, lse = run_decode(mla_problem(inp), 512, np_, 64)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "bf16 tiny np=%d" % np_)


@pytest.mark.parametrize("q_len", [1, 4])
def test_bf16_skipped_keys(q_len):
    lens = [900, 40, 3, 300]
    inp = workloads.mla_inputs(B=4, q_len=q_len, H=32, seq_lens=lens, pool_rows=1300, seed=161,
                               device=DEV, kv_dtype="bf16")
    gen = torch.Generator(device="cpu").manual_seed(161)
    idx = inp.kv_indices.cpu()
    idx[torch.rand(idx.shape, generator=gen) < 0.3] = -1
    a = int(inp.kv_indptr[2])
    idx[a:a + 3] = -1   # request 2: every key skipped
    inp.kv_indices = idx.to(DEV)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    for np_, bk in [(1, 64), (3, 32), (0, 0)]:
        log("bf16 skipped keys q_len=%d np=%d" % (q_len, np_))
        out, lse = run_decode(mla_problem(inp), 512, np_, bk)
        torch.cuda.synchronize()
        compare(out, lse, ref_o, ref_l, "bf16 skipped keys q_len=%d np=%d" % (q_len, np_))


@pytest.mark.parametrize("H,q_len", [(128, 1), (128, 2)])
def test_bf16_wide_head_counts(H, q_len):
    inp = workloads.mla_inputs(B=3, q_len=q_len, H=H, seq_lens=[2000, 65, 0], pool_rows=2100,
                               seed=166, device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    log("bf16 H=%d q_len=%d" % (H, q_len))
    out, lse = run_decode(mla_problem(inp), 512, 3, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "bf16 H=%d q_len=%d" % (H, q_len))


def test_bf16_context_parallel_ranks_merge_to_unsplit():
    from test_gpu_parity import dcp_rank_problem
    world, q_len = 3, 4
    inp = workloads.mla_inputs(B=4, q_len=q_len, H=16, seq_lens=[700, 5, 0, 1500], pool_rows=2300,
                               seed=191, device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    rows = inp.rows
    parts = torch.empty((world, rows, 512), dtype=torch.float32, device=DEV)
    lses = torch.empty((world, rows), dtype=torch.float32, device=DEV)
    for r in range(world):
        p = dcp_rank_problem(inp, world, r, inp.seq_lens)
        np_, bk = g.decode_plan(p)
        po = torch.empty((rows, np_, 512), dtype=torch.float32, device=DEV)
        pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
        g.decode_split(p, np_, bk, po, pl)
        g.splitk_reduce_f32(rows, np_, 512, po, pl, parts[r], lses[r])
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.merge_ranks(world, rows, 512, parts, lses, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "bf16 dcp world=%d" % world)


CASES = {
    "q_x32": lambda inp: workloads.scaled_queries(inp, 32.0),
    "q_rows_2^-20_to_8": lambda inp: workloads.wide_range_queries(inp, 20.0, 8.0, seed=21),
    "extreme_values": lambda inp: workloads.extreme_bf16_pool(inp, 0.15, 0.15, seed=22),
    "q_x8_extreme_values": lambda inp: workloads.extreme_bf16_pool(
        workloads.scaled_queries(inp, 8.0), seed=23),
    "dominant_key_per_tile": lambda inp: workloads.dominant_keys(inp, seed=24, block=32),
}


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("q_len", [1, 4])
def test_bf16_wide_dynamic_range(case, q_len):
    inp = CASES[case](workloads.mla_inputs(B=3, q_len=q_len, H=64, seq_lens=[2500, 700, 3],
                                           pool_rows=4000, seed=201 + q_len, device=DEV,
                                           kv_dtype="bf16"))
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp)
    planner_np, planner_bk = g.decode_plan(p)
    for np_, bk in ((1, 64), (planner_np, planner_bk)):
        what = "bf16 %s q_len=%d np=%d" % (case, q_len, np_)
        log("numerics " + what)
        o32, l32 = fp32_result(p, np_, bk)
        torch.cuda.synchronize()
        max_abs, rel, lse_err = compare(o32, l32, ref_o, ref_l, what + " fp32")
        out, lse = run_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        excess = compare_bf16_output(out, lse, ref_o, ref_l, what + " bf16")
        log("  fp32: max|dO| %.3g rel %.3g lse2 %.3g; bf16 excess %.3g" % (max_abs, rel, lse_err, excess))


def test_bf16_split_invariance_and_determinism():
    inp = workloads.mla_inputs(B=2, q_len=1, H=64, seq_lens=[5000, 3333], pool_rows=9000, seed=19,
                               device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    p = mla_problem(inp)
    base_o, base_l = run_decode(p, 512, 1, 64)
    for np_, bk in [(4, 32), (16, 64), (0, 0), (256, 32)]:
        o, l = run_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        assert (o.float() - base_o.float()).abs().max().item() <= 4e-3
        assert ((l - base_l).abs() / base_l.abs().clamp(min=1)).max().item() <= 1e-5
    o1, l1 = run_decode(p, 512, 16, 32)
    o2, l2 = run_decode(p, 512, 16, 32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


FULL = [("mla_b16_s131072_q1", lambda: workloads.mla_long_bf16(16, 1, DEV), 512),
        ("mla_b8_s131072_q4", lambda: workloads.mla_long_bf16(8, 4, DEV), 512),
        ("sparse_nq24", lambda: workloads.sparse_topk(24, DEV, kv_dtype="bf16"), 448),
        ("sparse_nq256", lambda: workloads.sparse_topk(256, DEV, kv_dtype="bf16"), 448)]


@pytest.mark.parametrize("name,make,d_v", FULL, ids=[n for n, _, _ in FULL])
def test_bf16_full_size_sampled(name, make, d_v):
    inp = make()
    torch.cuda.synchronize()
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("bf16 %s planner np=%d bk=%d" % (name, np_, bk))
    out, lse = run_decode(p, d_v)
    torch.cuda.synchronize()
    rows = sample_rows(inp.B, inp.q_len, inp.H, 24, seed=len(name))
    ref_o, ref_l = oracle_mla(inp, rows)
    compare(out[rows], lse[rows], ref_o, ref_l, "bf16 " + name)
    del inp, out, lse
    torch.cuda.empty_cache()


def test_bf16_other_entry_points():
    # the bf16 instance through decode_proportional (slot-major partials placed by the device
    # plan) and decode_scratch (partials in the static array), and 96 heads (a half row block)
    from test_gpu_proportional import run_prop
    from test_zz_no_alloc import scratch_decode
    lens = [9000, 0, 33, 1, 2500]
    inp = workloads.mla_inputs(B=5, q_len=1, H=96, seq_lens=lens, pool_rows=12000, seed=231,
                               device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp)
    log("bf16 proportional")
    out, lse = run_prop(p, 512, 8, 0, 32)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "bf16 proportional")
    log("bf16 scratch")
    d_o, d_l = run_decode(p, 512, 8, 32)
    s_o, s_l = scratch_decode(p, 512, 8, 32)
    torch.cuda.synchronize()
    assert torch.equal(s_o, d_o) and torch.equal(s_l, d_l)
    compare(s_o, s_l, ref_o, ref_l, "bf16 scratch")


def test_bf16_graph_replay_matches_eager():
    inp = workloads.mla_inputs(B=2, q_len=1, H=64, seq_lens=[3000, 700], pool_rows=4000, seed=241,
                               device=DEV, kv_dtype="bf16")
    torch.cuda.synchronize()
    p = mla_problem(inp)
    np_, bk = 8, 32
    out = torch.empty((p.rows, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((p.rows,), dtype=torch.float32, device=DEV)
    ws = torch.empty((g.decode_workspace_bytes(p, np_) // 4 + 64,), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()   # the inputs, built on the default stream, exist before `s` reads them
    with torch.cuda.stream(s):
        g.decode(p, out, lse, np=np_, block_k=bk, workspace=ws, stream=s)
    torch.cuda.synchronize()
    eager_o, eager_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.decode(p, out, lse, np=np_, block_k=bk, workspace=ws, stream=s)
    for _ in range(3):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l)


@pytest.mark.parametrize("np_,bk", [(1, 64), (3, 32), (0, 0)])
def test_bf16_second_cache(np_, bk):
    # ragged second-cache counts over a bf16 pool: none, fewer than a tile, tiles that straddle
    # the two caches, a whole list skipped, an extra list longer than the main one
    base = workloads.sparse_mla_inputs(num_queries=8, topk=200, cache_rows=4096, seed=4700,
                                       invalid_frac=0.1, device=DEV, kv_dtype="bf16")
    extra = [0, 7, 64, 100, 33, 1, 300, 129]
    skip = list(range(7, 7 + 64)) + [200, 201, 500]
    inp = workloads.with_second_cache(base, pool2_rows=2048, extra_lens=extra, seed=4710, skip=skip)
    torch.cuda.synchronize()
    assert inp.pool2.dtype == torch.bfloat16
    log("bf16 second cache np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(mla_problem(inp), 448, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "bf16 second cache np=%d bk=%d" % (np_, bk))


def test_bf16_second_cache_full_size():
    inp = workloads.sparse_mla_inputs(num_queries=32, seed=4800, extra_topk=512, device=DEV,
                                      kv_dtype="bf16")
    torch.cuda.synchronize()
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("bf16 second cache full size np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(p, 448, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp, n_threads=8)
    compare(out, lse, ref_o, ref_l, "bf16 second cache full size")


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("shape", ["one_head", "q_len16", "padded_rows"])
def test_mla_edge_shapes(kv, shape):
    # one query head (a 64-row block with one row), a 16-position draft window over 8 heads (two
    # row blocks per request), and a pool whose rows are padded (row stride 640 B for fp8 rows,
    # 1280 B for bf16 rows: a stride other than the row width)
    H, q_len, lens = {"one_head": (1, 1, [700, 5, 1]),
                      "q_len16": (8, 16, [900, 10, 300]),
                      "padded_rows": (64, 2, [1500, 66])}[shape]
    inp = workloads.mla_inputs(B=len(lens), q_len=q_len, H=H, seq_lens=lens, pool_rows=sum(lens) + 50,
                               seed=251, device=DEV, kv_dtype=kv)
    if shape == "padded_rows":
        width = inp.pool.shape[1]
        pad = torch.zeros((inp.pool.shape[0], width + 64), dtype=inp.pool.dtype, device=DEV)
        pad[:, :width] = inp.pool
        import dataclasses
        inp = dataclasses.replace(inp, pool=pad[:, :width])
        assert inp.pool.stride(0) == width + 64
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp)
    for np_, bk in ((1, 64), (0, 0)):
        log("edge %s %s np=%d" % (kv, shape, np_))
        out, lse = run_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        compare(out, lse, ref_o, ref_l, "edge %s %s np=%d" % (kv, shape, np_))
