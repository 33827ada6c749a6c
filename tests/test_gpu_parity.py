"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle, element by element.

Small shapes compare every output (several tiles, ragged tails, empty rows); the full-size
workloads compare sampled rows in exactly the launch configuration the benchmark times
(planner np, tile rule BLOCK_K)."""
import zlib
import numpy as np
import pytest
import torch

import gqa_plan_splits_amd as g
import oracle
import workloads
from gpu_util import (LSE_RTOL, OUT_ATOL, OUT_REL, compare, gqa_problem, log, mla_problem,
                      oracle_gqa, oracle_mla, run_decode, sample_rows)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


# ---------------------------------------------------------------------------------------------
# fp8 conversion and reducer
# ---------------------------------------------------------------------------------------------

def test_fp8_conversion_matches_definition():
    table = oracle.e4m3_table(False)
    src = torch.arange(256, dtype=torch.uint8, device=DEV).repeat(4)
    out = torch.empty(1024, dtype=torch.bfloat16, device=DEV)
    g.fp8_e4m3_to_bf16(src, 1024, out)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)[:256]
    ok = ~np.isnan(table)
    assert np.array_equal(got[ok], table[ok])
    assert np.all(np.isnan(got[~ok]))


@pytest.mark.parametrize("rows,np_,dv", [(1, 1, 512), (7, 2, 512), (33, 5, 448), (64, 64, 512),
                                         (10, 256, 128), (5, 37, 128), (300, 16, 512),
                                         (3, 13, 1024), (9, 250, 4), (128, 64, 512),
                                         (4100, 3, 448), (4500, 9, 1024)])
def test_reduce_matches_oracle_merge(rows, np_, dv):
    gen = torch.Generator(device="cpu").manual_seed(rows * 1000 + np_)
    po = torch.randn((rows, np_, dv), generator=gen) * 0.3
    pl = torch.randn((rows, np_), generator=gen) * 4 + 12
    drop = torch.rand((rows, np_), generator=gen) < 0.3
    pl[drop] = -float("inf")
    po[drop] = 0
    pl[0, :] = -float("inf")          # a row no partition saw
    po[0, :] = 0
    ref_o, ref_l = oracle.lse_merge(po.double().numpy(), pl.double().numpy())
    # a partition without weight is not read: NaN there must not reach the output
    po_dev = po.clone()
    po_dev[drop] = float("nan")
    po_dev[0, :] = float("nan")
    out = torch.empty((rows, dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce(rows, np_, dv, po_dev.to(DEV), pl.to(DEV), out, lse)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "reduce rows=%d np=%d dv=%d" % (rows, np_, dv))
    # bf16 output of an fp32 merge: within one bf16 rounding of the fp64 merge
    o = out.float().cpu().double().numpy()
    assert np.all(np.abs(o - ref_o) <= np.abs(ref_o) * 2 ** -8 + 1e-6)


def test_reduce_f32_output_matches_oracle_merge():
    gen = torch.Generator(device="cpu").manual_seed(17)
    rows, np_, dv = 40, 24, 512
    po = torch.randn((rows, np_, dv), generator=gen) * 0.3
    pl = torch.randn((rows, np_), generator=gen) * 4 + 12
    pl[2, :] = -float("inf")
    po[2, :] = 0
    ref_o, ref_l = oracle.lse_merge(po.double().numpy(), pl.double().numpy())
    out = torch.empty((rows, dv), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce_f32(rows, np_, dv, po.to(DEV), pl.to(DEV), out, lse)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    # an fp32 merge: far inside the bf16 bar
    assert np.all(o[2] == 0) and np.isneginf(lse[2].item())
    assert np.abs(o - ref_o).max() <= 1e-5
    ok = ~np.isinf(ref_l)
    assert np.all(np.abs(lse.cpu().double().numpy()[ok] - ref_l[ok]) <= 1e-5 * np.maximum(1, np.abs(ref_l[ok])))


def test_reduce_is_deterministic():
    po = torch.randn((64, 200, 512), device=DEV)
    pl = torch.randn((64, 200), device=DEV) * 3
    outs = []
    for _ in range(3):
        out = torch.empty((64, 512), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((64,), dtype=torch.float32, device=DEV)
        g.splitk_reduce(64, 200, 512, po, pl, out, lse)
        outs.append((out.clone(), lse.clone()))
    torch.cuda.synchronize()
    for o, l in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(l, outs[0][1])


# ---------------------------------------------------------------------------------------------
# Absorbed MLA
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("np_", [1, 4, 16, 0])
@pytest.mark.parametrize("bk", [32, 64])
def test_mla_tiny_all_rows(np_, bk):
    inp = workloads.mla_tiny(DEV)
    log("mla tiny np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(mla_problem(inp), 512, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "mla tiny np=%d bk=%d" % (np_, bk))


@pytest.mark.parametrize("d_qk,d_v", [(576, 512), (512, 448)])
@pytest.mark.parametrize("q_len", [1, 3, 4])
@pytest.mark.parametrize("np_", [1, 3, 8])
@pytest.mark.parametrize("bk", [32, 64])
def test_mla_ragged_all_rows(d_qk, d_v, q_len, np_, bk):
    # several tiles per partition, ragged tails, a request shorter than the draft window (rows
    # that see no key), an empty request, and 40 heads (a partial second 32-row block; q_len 3:
    # 120 rows per request, a partial second 64-row block)
    lens = [1000, 37, 2, 0, 2049]
    inp = workloads.mla_inputs(B=5, q_len=q_len, H=40, seq_lens=lens, pool_rows=4000, d_qk=d_qk,
                               d_v=d_v, seed=77, device=DEV, fused_q=(d_qk == 512))
    log("mla ragged d_qk=%d q_len=%d np=%d bk=%d" % (d_qk, q_len, np_, bk))
    out, lse = run_decode(mla_problem(inp), d_v, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "mla ragged")


def test_mla_split_partials_match_oracle_on_key_ranges():
    # decode_split alone: each partial equals the oracle over that partition's key range
    inp = workloads.mla_inputs(B=2, q_len=1, H=32, seq_lens=[300, 129], pool_rows=512, seed=5,
                               device=DEV)
    np_, bk = 3, 32
    p = mla_problem(inp)
    rows = inp.rows
    po = torch.empty((rows, np_, 512), dtype=torch.float32, device=DEV)
    pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
    g.decode_split(p, np_, bk, po, pl)
    torch.cuda.synchronize()
    for b, S in enumerate([300, 129]):
        chunk = -(-(-(-S // np_)) // bk) * bk
        for part in range(np_):
            a, e = min(S, part * chunk), min(S, (part + 1) * chunk)
            sub = workloads.mla_inputs(B=1, q_len=1, H=32, seq_lens=[1], pool_rows=1, seed=5)
            sub.q_lat = inp.q_lat[b:b + 1].cpu()
            sub.q_pe = inp.q_pe[b:b + 1].cpu()
            sub.pool = inp.pool.cpu()
            base = int(inp.kv_indptr[b])
            sub.kv_indices = inp.kv_indices[base + a:base + max(e, a + 1)].cpu()
            sub.kv_indptr = torch.tensor([0, max(e - a, 1)], dtype=torch.int32)
            sub.seq_lens = torch.tensor([e - a], dtype=torch.int32)
            sub.B = 1
            ro, rl = oracle_mla(sub)
            got_o = po[b * 32:(b + 1) * 32, part].cpu().double().numpy()
            got_l = pl[b * 32:(b + 1) * 32, part].cpu().double().numpy()
            if e <= a:
                assert np.all(got_l == -np.inf) and np.all(got_o == 0)
                continue
            # the same bar as every output (fp32 partials; bf16 rounding of P bounds the error)
            err = np.abs(got_o - ro).max()
            assert err <= OUT_ATOL and err <= OUT_REL * np.abs(ro).max()
            assert np.all(np.abs(got_l - rl) <= LSE_RTOL * np.maximum(1, np.abs(rl)))


@pytest.mark.parametrize("q_len", [1, 4])
def test_mla_skipped_keys_match_oracle(q_len):
    # negative slot ids (the top-k lists' has_invalid case) are keys with no weight; request 2's
    # list is all -1
    lens = [900, 40, 3, 300]
    inp = workloads.mla_inputs(B=4, q_len=q_len, H=32, seq_lens=lens, pool_rows=1300, seed=61,
                               device=DEV)
    gen = torch.Generator(device="cpu").manual_seed(61)
    idx = inp.kv_indices.cpu()
    idx[torch.rand(idx.shape, generator=gen) < 0.3] = -1
    a = int(inp.kv_indptr[2])
    idx[a:a + 3] = -1
    inp.kv_indices = idx.to(DEV)
    ref_o, ref_l = oracle_mla(inp)
    for np_, bk in [(1, 64), (3, 32), (0, 0)]:
        log("mla skipped keys q_len=%d np=%d bk=%d" % (q_len, np_, bk))
        out, lse = run_decode(mla_problem(inp), 512, np_, bk)
        torch.cuda.synchronize()
        compare(out, lse, ref_o, ref_l, "mla skipped keys q_len=%d np=%d" % (q_len, np_))


@pytest.mark.parametrize("H,q_len", [(128, 1), (128, 2), (96, 1)])
@pytest.mark.parametrize("np_", [1, 3])
def test_mla_wide_head_counts_match_oracle(H, q_len, np_):
    # more than one 64-row block per request from the heads alone (and a half block at 96)
    inp = workloads.mla_inputs(B=3, q_len=q_len, H=H, seq_lens=[2000, 65, 0], pool_rows=2100,
                               seed=66, device=DEV)
    torch.cuda.synchronize()
    log("mla H=%d q_len=%d np=%d" % (H, q_len, np_))
    out, lse = run_decode(mla_problem(inp), 512, np_, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "mla H=%d q_len=%d np=%d" % (H, q_len, np_))


def test_sparse_skipped_keys_match_oracle():
    inp = workloads.sparse_mla_inputs(num_queries=24, invalid_frac=0.25, all_invalid=(5,), seed=4100,
                                      device=DEV)
    log("sparse skipped keys")
    out, lse = run_decode(mla_problem(inp), 448)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "sparse skipped keys")
    assert torch.all(lse[5 * 64:6 * 64] == -float("inf"))


@pytest.mark.parametrize("np_,bk", [(1, 64), (3, 32), (5, 64), (0, 0)])
def test_sparse_second_cache_matches_oracle(np_, bk):
    # ragged second-cache counts: none, fewer than a tile, tiles that straddle the boundary
    # between the caches, a whole list skipped, an extra list longer than the main one
    base = workloads.sparse_mla_inputs(num_queries=8, topk=200, cache_rows=4096, seed=4300,
                                       invalid_frac=0.1, device=DEV)
    extra = [0, 7, 64, 100, 33, 1, 300, 129]
    skip = list(range(7, 7 + 64)) + [200, 201, 500]
    inp = workloads.with_second_cache(base, pool2_rows=2048, extra_lens=extra, seed=4310, skip=skip)
    torch.cuda.synchronize()
    log("sparse second cache np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(mla_problem(inp), 448, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "sparse second cache np=%d bk=%d" % (np_, bk))


def test_sparse_second_cache_only():
    # every main key skipped: the second cache alone decides the output; a request with both
    # lists skipped stays empty
    base = workloads.sparse_mla_inputs(num_queries=4, topk=96, cache_rows=1024, seed=4400,
                                       all_invalid=(0, 1, 2, 3), device=DEV)
    inp = workloads.with_second_cache(base, pool2_rows=1024, extra_lens=[150, 64, 0, 5], seed=4410,
                                      skip=list(range(214, 219)))
    torch.cuda.synchronize()
    log("sparse second cache only")
    out, lse = run_decode(mla_problem(inp), 448, 2, 64)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "sparse second cache only")
    assert torch.all(lse[2 * 64:4 * 64] == -float("inf"))


def test_sparse_second_cache_full_size():
    # the sparse workload at 32 queries with 512 extra candidates per query, planner launch
    inp = workloads.sparse_mla_inputs(num_queries=32, seed=4500, extra_topk=512, device=DEV)
    torch.cuda.synchronize()
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("sparse second cache full size np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(p, 448, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp, n_threads=8)
    compare(out, lse, ref_o, ref_l, "sparse second cache full size")


def dcp_rank_problem(inp, world, rank, glen):
    """Rank `rank` of `world` decode-context-parallel ranks: the positions p % world == rank of
    every request (in position order), with the global lengths in glen."""
    idx = inp.kv_indices.cpu()
    indptr = inp.kv_indptr.cpu()
    lens = inp.seq_lens.cpu()
    parts, new_lens, new_indptr = [], [], [0]
    for b in range(inp.B):
        a, S = int(indptr[b]), int(lens[b])
        sel = idx[a + rank:a + S:world]
        parts.append(sel)
        new_lens.append(len(sel))
        new_indptr.append(new_indptr[-1] + len(sel))
    kv_idx = torch.cat(parts) if new_indptr[-1] else torch.zeros(1, dtype=torch.int32)
    kv_idx = kv_idx.to(DEV)
    kv_indptr = torch.tensor(new_indptr, dtype=torch.int32, device=DEV)
    seq = torch.tensor(new_lens, dtype=torch.int32, device=DEV)
    return g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, kv_idx, kv_indptr, seq, batch=inp.B,
                         q_len=inp.q_len, num_heads=inp.H, max_num_keys=max(new_lens),
                         scale=inp.scale, kv_scale=inp.kv_scale, d_v=inp.d_v, glen=glen,
                         cp_rank=rank, cp_world=world)


@pytest.mark.parametrize("world", [2, 3, 8])
@pytest.mark.parametrize("q_len", [1, 4])
def test_mla_context_parallel_ranks_merge_to_unsplit(world, q_len):
    # each rank decodes its interleaved share of the positions (window on global positions);
    # merging the ranks' outputs equals attention over the whole sequence
    lens = [700, 5, 0, 1500, 3]
    inp = workloads.mla_inputs(B=5, q_len=q_len, H=16, seq_lens=lens, pool_rows=2300, seed=91,
                               device=DEV)
    log("mla dcp world=%d q_len=%d" % (world, q_len))
    rows = inp.rows
    parts = torch.empty((world, rows, 512), dtype=torch.float32, device=DEV)
    lses = torch.empty((world, rows), dtype=torch.float32, device=DEV)
    for r in range(world):
        # each rank: its split, then its own merge to an fp32 output
        p = dcp_rank_problem(inp, world, r, inp.seq_lens)
        np_, bk = g.decode_plan(p, 0 if r % 2 else 4, 0 if r % 2 else 32)
        po = torch.empty((rows, np_, 512), dtype=torch.float32, device=DEV)
        pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
        g.decode_split(p, np_, bk, po, pl)
        g.splitk_reduce_f32(rows, np_, 512, po, pl, parts[r], lses[r])
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.merge_ranks(world, rows, 512, parts, lses, out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "mla dcp world=%d q_len=%d" % (world, q_len))


def test_merge_ranks_matches_oracle_merge():
    gen = torch.Generator(device="cpu").manual_seed(5)
    world, rows, dv = 6, 70, 512
    parts = torch.randn((world, rows, dv), generator=gen) * 0.3
    lses = torch.randn((world, rows), generator=gen) * 4 + 12
    lses[torch.rand((world, rows), generator=gen) < 0.3] = -float("inf")
    lses[:, 3] = -float("inf")   # a row no rank saw
    po = parts.double().numpy().transpose(1, 0, 2).copy()
    pl = lses.double().numpy().T.copy()
    po[np.isinf(pl)] = 0
    ref_o, ref_l = oracle.lse_merge(po, pl)
    dev_parts = parts.clone()
    dev_parts[torch.isinf(lses)] = float("nan")   # a rank without weight is not read
    out = torch.empty((rows, dv), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.merge_ranks(world, rows, dv, dev_parts.to(DEV), lses.to(DEV), out, lse)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "merge_ranks")


def test_mla_split_invariance_and_determinism():
    inp = workloads.mla_inputs(B=2, q_len=1, H=64, seq_lens=[5000, 3333], pool_rows=9000, seed=9,
                               device=DEV)
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


def test_mla_graph_replay_matches_eager():
    inp = workloads.mla_inputs(B=2, q_len=2, H=64, seq_lens=[4000, 2500], pool_rows=7000, seed=3,
                               device=DEV)
    p = mla_problem(inp)
    rows = inp.rows
    ws = torch.empty((g.decode_workspace_bytes(p, 8) // 4 + 64,), dtype=torch.float32, device=DEV)
    out = torch.empty((rows, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()   # the inputs, built on the default stream, exist before `s` reads them
    with torch.cuda.stream(s):
        g.decode(p, out, lse, np=8, block_k=32, workspace=ws, stream=s)
    torch.cuda.synchronize()
    eager_o, eager_l = out.clone(), lse.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.decode(p, out, lse, np=8, block_k=32, workspace=ws, stream=s)
    for _ in range(4):
        out.zero_()
        lse.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_o) and torch.equal(lse, eager_l)


def test_graph_replay_with_new_lengths():
    # the partition count is fixed when the graph is captured (from the host-known maximum);
    # lengths, index lists and windows are read on the device at every replay, so one captured
    # decode serves new lengths with no host work
    lens_a, lens_b = [3000, 700, 1500], [2999, 0, 2048]
    inp = workloads.mla_inputs(B=3, q_len=2, H=64, seq_lens=lens_a, pool_rows=6000, seed=71,
                               device=DEV)
    inp_b = workloads.mla_inputs(B=3, q_len=2, H=64, seq_lens=lens_b, pool_rows=6000, seed=72,
                                 device=DEV)
    # the new index list must fit the captured buffer: pad it to the old length
    idx = torch.zeros_like(inp.kv_indices)
    idx[:inp_b.kv_indices.numel()] = inp_b.kv_indices
    p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr, inp.seq_lens,
                      batch=3, q_len=2, num_heads=64, max_num_keys=3000, scale=inp.scale,
                      kv_scale=inp.kv_scale, d_v=512)
    np_, bk = g.decode_plan(p)
    ws = torch.empty((g.decode_workspace_bytes(p, np_) // 4 + 64,), dtype=torch.float32, device=DEV)
    out = torch.empty((inp.rows, 512), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((inp.rows,), dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()   # the inputs, built on the default stream, exist before `s` reads them
    with torch.cuda.stream(s):
        g.decode(p, out, lse, np=np_, block_k=bk, workspace=ws, stream=s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.decode(p, out, lse, np=np_, block_k=bk, workspace=ws, stream=s)
    # the lengths-a and lengths-b contents of the captured buffers
    data = {False: (inp.q_lat.clone(), inp.q_pe.clone(), inp.pool.clone(), inp.kv_indices.clone(),
                    inp.kv_indptr.clone(), inp.seq_lens.clone()),
            True: (inp_b.q_lat, inp_b.q_pe, inp_b.pool, idx, inp_b.kv_indptr, inp_b.seq_lens)}
    refs = {False: oracle_mla(inp), True: oracle_mla(inp_b)}
    for new in (True, False, True):
        for dst, src in zip((inp.q_lat, inp.q_pe, inp.pool, inp.kv_indices, inp.kv_indptr,
                             inp.seq_lens), data[new]):
            dst.copy_(src)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = refs[new]
        compare(out, lse, ref_o, ref_l, "graph replay lengths %s" % (lens_b if new else lens_a))


FULL_MLA = [("b2_s65536", lambda: workloads.mla_b2_s65536(DEV)),
            ("b8_s131072_q1", lambda: workloads.mla_long(8, 1, DEV)),
            ("b16_s131072_q1", lambda: workloads.mla_long(16, 1, DEV)),
            ("b8_s131072_q4", lambda: workloads.mla_long(8, 4, DEV)),
            ("b16_s131072_q4", lambda: workloads.mla_long(16, 4, DEV))]


@pytest.mark.parametrize("name,make", FULL_MLA, ids=[n for n, _ in FULL_MLA])
def test_mla_full_size_sampled(name, make):
    inp = make()
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("mla %s planner np=%d bk=%d" % (name, np_, bk))
    out, lse = run_decode(p, 512)
    torch.cuda.synchronize()
    # 128 rows (a stable seed per workload: str hashes vary between processes)
    rows = sample_rows(inp.B, inp.q_len, inp.H, 128, seed=zlib.crc32(name.encode()) % 1000)
    ref_o, ref_l = oracle_mla(inp, rows)
    compare(out[rows], lse[rows], ref_o, ref_l, "mla " + name)
    del inp, out, lse
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------------------------
# Sparse top-k MLA
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("nq", list(workloads.SPARSE_QUERY_COUNTS))
def test_sparse_full_size_both_tiles(nq):
    inp = workloads.sparse_topk(nq, DEV)
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("sparse nq=%d planner np=%d bk=%d" % (nq, np_, bk))
    rows = sample_rows(inp.B, 1, inp.H, 128, seed=nq)
    ref_o, ref_l = oracle_mla(inp, rows)
    results = {}
    for tile in (32, 64):   # the rule's choice and the other one: same numerics either way
        out, lse = run_decode(p, 448, np_, tile)
        torch.cuda.synchronize()
        compare(out[rows], lse[rows], ref_o, ref_l, "sparse nq=%d bk=%d" % (nq, tile))
        results[tile] = (out, lse)
    d = (results[32][0].float() - results[64][0].float()).abs().max().item()
    assert d <= 4e-3


# ---------------------------------------------------------------------------------------------
# Paged GQA
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("Hq,Hkv,q_len", [(16, 2, 1), (32, 4, 2), (8, 8, 1), (12, 3, 4), (16, 1, 1)])
@pytest.mark.parametrize("np_", [1, 3, 32])
@pytest.mark.parametrize("bk", [32, 64])
def test_gqa_ragged_all_rows(Hq, Hkv, q_len, np_, bk):
    lens = [700, 33, 1, 0, 1600, 16]
    inp = workloads.gqa_inputs(B=6, Hq=Hq, Hkv=Hkv, D=128, page_size=16, seq_lens=lens,
                               num_pages=300, q_len=q_len, seed=31, device=DEV)
    log("gqa ragged Hq=%d Hkv=%d q_len=%d np=%d bk=%d" % (Hq, Hkv, q_len, np_, bk))
    out, lse = run_decode(gqa_problem(inp), 128, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa ragged")


# More than 16 query rows per kv head: 17 to 32 rows run 2 waves of 16 rows over each tile, 33 to
# 64 rows 2 waves of 32 rows.
# Shapes: 64 heads on one kv head (MQA), 24 rows (a half-empty second block), 30 rows where a
# draft position straddles two blocks, 51 rows (the second 32-row wave holds 19), 64 rows from
# q_len 8 x 8.
@pytest.mark.parametrize("Hq,Hkv,q_len", [(64, 1, 1), (24, 1, 1), (20, 2, 3), (17, 1, 3),
                                          (64, 8, 8), (32, 1, 2)])
@pytest.mark.parametrize("np_,bk", [(1, 32), (3, 64), (32, 32), (0, 0)])
def test_gqa_row_blocks_all_rows(Hq, Hkv, q_len, np_, bk):
    lens = [700, 33, 1, 0, 1600, 16]
    inp = workloads.gqa_inputs(B=6, Hq=Hq, Hkv=Hkv, D=128, page_size=16, seq_lens=lens,
                               num_pages=300, q_len=q_len, seed=33, device=DEV)
    log("gqa row blocks Hq=%d Hkv=%d q_len=%d np=%d bk=%d" % (Hq, Hkv, q_len, np_, bk))
    out, lse = run_decode(gqa_problem(inp), 128, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa row blocks")


# The most partitions a call allows (256): most partitions of the short requests are empty and the
# others hold one tile or a partial one; the pair kernel (16 rows), two 16-row waves (24 rows)
# and two 32-row waves (48 rows), through decode and through decode_split + splitk_reduce_f32.
@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (24, 1), (48, 1)])
def test_gqa_max_partitions(Hq, Hkv):
    lens = [9000, 100, 0, 33, 2600]
    pages = sum(-(-L // 16) for L in lens)
    inp = workloads.gqa_inputs(B=5, Hq=Hq, Hkv=Hkv, D=128, page_size=16, seq_lens=lens,
                               num_pages=pages + 3, q_len=1, seed=47, device=DEV)
    p = gqa_problem(inp)
    ref_o, ref_l = oracle_gqa(inp)
    log("gqa np=256 Hq=%d Hkv=%d" % (Hq, Hkv))
    out, lse = run_decode(p, 128, 256, 32)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "gqa np=256 decode")
    po = torch.empty((p.rows, 256, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((p.rows, 256), dtype=torch.float32, device=DEV)
    g.decode_split(p, 256, 32, po, pl)
    o32 = torch.empty((p.rows, 128), dtype=torch.float32, device=DEV)
    l32 = torch.empty((p.rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce_f32(p.rows, 256, 128, po, pl, o32, l32)
    torch.cuda.synchronize()
    compare(o32, l32, ref_o, ref_l, "gqa np=256 split + reduce")


# 33 to 64 rows run on 32-row waves with 32-token tiles: a tile covers four pages of 8 tokens,
# two of 16 or part of one of 64; 40 rows leave the second wave's rows 40-63 empty.
@pytest.mark.parametrize("page_size", [8, 16, 64])
@pytest.mark.parametrize("np_,bk", [(1, 32), (5, 64), (0, 0)])
def test_gqa_rows32_page_sizes(page_size, np_, bk):
    lens = [1333, 64, 0, 31, 2000]
    pages = sum(-(-L // page_size) for L in lens)
    inp = workloads.gqa_inputs(B=5, Hq=40, Hkv=1, D=128, page_size=page_size, seq_lens=lens,
                               num_pages=pages + 11, q_len=1, seed=45, device=DEV)
    log("gqa 40 rows page=%d np=%d bk=%d" % (page_size, np_, bk))
    out, lse = run_decode(gqa_problem(inp), 128, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa 40 rows page %d" % page_size)


def test_gqa_row_blocks_other_entry_points():
    # the scratch and proportional entry points launch the same kernel with other partial layouts
    lens = [9000, 31, 0, 2500, 700]
    inp = workloads.gqa_inputs(B=5, Hq=48, Hkv=1, D=128, page_size=32, seq_lens=lens,
                               num_pages=420, q_len=1, seed=35, device=DEV)
    p = gqa_problem(inp)
    ref_o, ref_l = oracle_gqa(inp)
    log("gqa row blocks scratch")
    out = torch.empty((p.rows, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((p.rows,), dtype=torch.float32, device=DEV)
    g.decode_scratch(p, out, lse, np=6, block_k=32)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "gqa row blocks scratch")
    log("gqa row blocks proportional")
    nbytes = g.decode_proportional_workspace_bytes(p, 12, 0)
    ws = torch.empty((nbytes // 4 + 64,), dtype=torch.float32, device=DEV)
    g.decode_proportional(p, out, lse, np=12, cap=0, block_k=32, workspace=ws)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "gqa row blocks proportional")


def test_gqa_mqa_full_size_sampled():
    # 64 query heads over one kv head, 32 requests of 32768 tokens, planner launch
    lens = [32768] * 32
    inp = workloads.gqa_inputs(B=32, Hq=64, Hkv=1, D=128, page_size=16, seq_lens=lens,
                               num_pages=32 * 2048, seed=37, device=DEV)
    p = gqa_problem(inp)
    np_, bk = g.decode_plan(p)
    log("gqa mqa full planner np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(p, 128)
    torch.cuda.synchronize()
    rows = sample_rows(inp.B, 1, inp.Hq, 128, seed=124)
    ref_o, ref_l = oracle_gqa(inp, rows)
    compare(out[rows], lse[rows], ref_o, ref_l, "gqa mqa full")
    o2, l2 = run_decode(p, 128)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)


# An even number of kv heads with up to 16 query rows per head group: a CTA serves a pair of kv
# heads and copies both heads' rows of each token as one run.  Shapes: 16 and 24 kv heads (8 and
# 12 CTAs per request and partition, the last pair at heads 14-15 and 22-23), 16 rows from
# q_len 2 x 8, 15 rows from q_len 5 x 3, pages of 8 tokens (each tile on two pages) and of 64.
@pytest.mark.parametrize("Hq,Hkv,q_len,page_size", [(32, 16, 1, 16), (48, 24, 2, 16), (64, 8, 2, 8),
                                                    (12, 4, 5, 64), (4, 2, 1, 8), (128, 16, 1, 32)])
@pytest.mark.parametrize("np_,bk", [(1, 32), (5, 64), (32, 32), (0, 0)])
def test_gqa_kv_head_pairs(Hq, Hkv, q_len, page_size, np_, bk):
    lens = [700, 33, 1, 0, 1600, 16]
    pages = sum(-(-L // page_size) for L in lens)
    inp = workloads.gqa_inputs(B=6, Hq=Hq, Hkv=Hkv, D=128, page_size=page_size, seq_lens=lens,
                               num_pages=pages + 9, q_len=q_len, seed=39, device=DEV)
    log("gqa head pairs Hq=%d Hkv=%d q_len=%d page=%d np=%d bk=%d" % (Hq, Hkv, q_len, page_size, np_, bk))
    out, lse = run_decode(gqa_problem(inp), 128, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa head pairs")


def test_gqa_kv_head_pairs_other_entry_points():
    lens = [9000, 31, 0, 2500, 700]
    inp = workloads.gqa_inputs(B=5, Hq=64, Hkv=16, D=128, page_size=32, seq_lens=lens,
                               num_pages=420, q_len=1, seed=43, device=DEV)
    p = gqa_problem(inp)
    ref_o, ref_l = oracle_gqa(inp)
    log("gqa head pairs scratch")
    out = torch.empty((p.rows, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((p.rows,), dtype=torch.float32, device=DEV)
    g.decode_scratch(p, out, lse, np=6, block_k=32)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "gqa head pairs scratch")
    log("gqa head pairs proportional")
    nbytes = g.decode_proportional_workspace_bytes(p, 12, 0)
    ws = torch.empty((nbytes // 4 + 64,), dtype=torch.float32, device=DEV)
    g.decode_proportional(p, out, lse, np=12, cap=0, block_k=32, workspace=ws)
    torch.cuda.synchronize()
    compare(out, lse, ref_o, ref_l, "gqa head pairs proportional")


# The one-head kernel with 16-row waves at other page sizes: one wave (3 kv heads, 12 rows each
# at q_len 4) and two waves (24 rows on one kv head); a tile covers two pages of 8 tokens or part
# of one of 64.
@pytest.mark.parametrize("Hq,Hkv,q_len", [(9, 3, 4), (24, 1, 1)])
@pytest.mark.parametrize("page_size", [8, 64])
def test_gqa_one_head_page_sizes(Hq, Hkv, q_len, page_size):
    lens = [1333, 64, 0, 31, 2000]
    pages = sum(-(-L // page_size) for L in lens)
    inp = workloads.gqa_inputs(B=5, Hq=Hq, Hkv=Hkv, D=128, page_size=page_size, seq_lens=lens,
                               num_pages=pages + 11, q_len=q_len, seed=49, device=DEV)
    ref_o, ref_l = oracle_gqa(inp)
    for np_, bk in ((1, 32), (6, 64), (0, 0)):
        log("gqa one head Hq=%d Hkv=%d q_len=%d page=%d np=%d" % (Hq, Hkv, q_len, page_size, np_))
        out, lse = run_decode(gqa_problem(inp), 128, np_, bk)
        torch.cuda.synchronize()
        compare(out, lse, ref_o, ref_l, "gqa one head page %d" % page_size)


@pytest.mark.parametrize("page_size", [8, 32, 64])
def test_gqa_page_sizes(page_size):
    lens = [333, 64, 1000]
    pages = sum(-(-L // page_size) for L in lens)
    inp = workloads.gqa_inputs(B=3, Hq=16, Hkv=2, D=128, page_size=page_size, seq_lens=lens,
                               num_pages=pages + 7, seed=41, device=DEV)
    out, lse = run_decode(gqa_problem(inp), 128, 4, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa page %d" % page_size)


@pytest.mark.parametrize("B", [20, 64, 70])
def test_gqa_batch_order(B):
    # CTAs take requests longest first (batches of up to 64): tied lengths, empty requests and a
    # batch past 64 (kept in its own order) must all land on the right rows
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.choice([0, 5, 16, 17, 90, 90, 90, 250, 251], size=B)]
    pages = sum(-(-L // 16) for L in lens)
    inp = workloads.gqa_inputs(B=B, Hq=8, Hkv=2, D=128, page_size=16, seq_lens=lens,
                               num_pages=pages + 5, seed=57 + B, device=DEV)
    log("gqa batch order B=%d" % B)
    for np_ in (1, 4):
        out, lse = run_decode(gqa_problem(inp), 128, np_, 32)
        torch.cuda.synchronize()
        ref_o, ref_l = oracle_gqa(inp)
        compare(out, lse, ref_o, ref_l, "gqa batch order B=%d np=%d" % (B, np_))


def test_gqa_full_size_sampled():
    inp = workloads.gqa_paged(DEV)
    p = gqa_problem(inp)
    np_, bk = g.decode_plan(p)
    log("gqa full planner np=%d bk=%d" % (np_, bk))
    out, lse = run_decode(p, 128)
    torch.cuda.synchronize()
    rows = sample_rows(inp.B, 1, inp.Hq, 48, seed=123)
    ref_o, ref_l = oracle_gqa(inp, rows)
    compare(out[rows], lse[rows], ref_o, ref_l, "gqa full")
    o2, l2 = run_decode(p, 128)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
