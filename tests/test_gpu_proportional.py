"""GPU parity of the device-side length-proportional plan and of decode_proportional.

The plan tables are compared bit-exactly with the oracle's rule; the decode output is compared
element by element with the fp64 attention oracle (the partitioning changes only rounding)."""
import numpy as np
import pytest
import torch

import gqa_plan_splits_amd as g
import oracle
import workloads
from gpu_util import compare, gqa_problem, log, mla_problem, oracle_gqa, oracle_mla

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def run_prop(problem, d_v, np_=0, cap=0, bk=0, stream=None, ws=None):
    rows = problem.rows
    out = torch.empty((rows, d_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    if ws is None:
        nbytes = g.decode_proportional_workspace_bytes(problem, np_, cap)
        ws = torch.empty((nbytes // 4 + 64,), dtype=torch.float32, device=DEV)
        ws.fill_(float("nan"))   # a slot the plan leaves unmarked would show up as NaN
    g.decode_proportional(problem, out, lse, np=np_, cap=cap, block_k=bk, workspace=ws, stream=stream)
    return out, lse


PLAN_CASES = [
    ("ragged", [1000, 0, 31, 5000], 8, 4, 32, None),
    ("uniform", [65536, 65536], 128, 256, 32, None),
    ("one long", [17] * 40 + [300000] + [5] * 30, 71 * 3, 64, 64, None),
    ("all empty", [0, 0, 0], 9, 8, 32, None),
    ("wide batch", None, 600 * 2, 8, 32, None),          # 600 requests: three scan rounds
    ("second cache", [100, 2048, 0, 7], 16, 16, 64, [0, 64, 64, 1000, 1001]),
    ("past the LDS cache", "big", 9000 * 2, 16, 32, None),   # 9000 requests: counts read from memory
    # key counts at the int32 edge (held to 2^31 - 64, so that every chunk fits an int32): with
    # cap 1 each request's chunk is its whole length rounded up to block_k
    ("near 2^31", [2 ** 31 - 1, 2 ** 31 - 40, 5, 0], 3, 1, 64, None),
    ("near 2^31 with a second cache", [2 ** 31 - 100, 7], 2, 1, 32, [0, 200, 201]),
]
MAX_KEYS = 2 ** 31 - 64


@pytest.mark.parametrize("name,lens,budget,cap,bk,extra", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_plan_tables_match_oracle(name, lens, budget, cap, bk, extra):
    if lens is None:
        lens = np.random.default_rng(5).integers(0, 40000, 600).tolist()
    elif lens == "big":
        lens = np.random.default_rng(6).integers(0, 3000, 9000).tolist()
    B = len(lens)
    log("proportional plan %s B=%d budget=%d cap=%d bk=%d" % (name, B, budget, cap, bk))
    seq = torch.tensor(lens, dtype=torch.int32, device=DEV)
    ext = None if extra is None else torch.tensor(extra, dtype=torch.int32, device=DEV)
    start = torch.full((B + 1,), -7, dtype=torch.int32, device=DEV)
    chunk = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    g.plan_proportional_device(seq, ext, B, budget, cap, bk, start, chunk)
    torch.cuda.synchronize()
    keys = list(lens) if extra is None else [lens[b] + extra[b + 1] - extra[b] for b in range(B)]
    ref_start, ref_chunk = oracle.proportional_plan([min(k, MAX_KEYS) for k in keys], budget, cap, bk)
    assert start.cpu().tolist() == ref_start
    assert chunk.cpu().tolist() == ref_chunk


@pytest.mark.parametrize("q_len", [1, 4])
@pytest.mark.parametrize("np_,cap", [(2, 0), (4, 3), (16, 64), (1, 1)])
def test_mla_proportional_matches_oracle(q_len, np_, cap):
    lens = [9000, 0, 33, 1, 2500, 64, 700]
    inp = workloads.mla_inputs(B=7, q_len=q_len, H=64, seq_lens=lens, pool_rows=16000, seed=81,
                               device=DEV)
    torch.cuda.synchronize()
    log("mla proportional q_len=%d np=%d cap=%d" % (q_len, np_, cap))
    out, lse = run_prop(mla_problem(inp), 512, np_, cap, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "mla proportional q_len=%d np=%d cap=%d" % (q_len, np_, cap))


def test_sparse_proportional_with_second_cache():
    base = workloads.sparse_mla_inputs(num_queries=8, topk=200, cache_rows=4096, seed=4600,
                                       invalid_frac=0.1, device=DEV)
    inp = workloads.with_second_cache(base, pool2_rows=2048, extra_lens=[0, 7, 64, 1000, 33, 1, 300, 129],
                                      seed=4610, skip=[3, 4, 500])
    torch.cuda.synchronize()
    log("sparse proportional second cache")
    out, lse = run_prop(mla_problem(inp), 448, 2, 0, 64)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "sparse proportional second cache")


@pytest.mark.parametrize("B,q_len,np_", [(6, 1, 3), (6, 2, 8), (70, 1, 2)])
def test_gqa_proportional_matches_oracle(B, q_len, np_):
    rng = np.random.default_rng(B * 10 + q_len)
    lens = rng.integers(0, 3000, B).tolist()
    lens[0], lens[-1] = 9000, 0
    pages = sum((n + 15) // 16 for n in lens) + 8
    inp = workloads.gqa_inputs(B=B, Hq=16, Hkv=2, D=128, page_size=16, seq_lens=lens,
                               num_pages=pages, q_len=q_len, seed=91, device=DEV)
    torch.cuda.synchronize()
    log("gqa proportional B=%d q_len=%d np=%d" % (B, q_len, np_))
    out, lse = run_prop(gqa_problem(inp), 128, np_, 0, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_gqa(inp)
    compare(out, lse, ref_o, ref_l, "gqa proportional B=%d q_len=%d" % (B, q_len))


def test_proportional_graph_replays_with_new_lengths():
    # one captured decode_proportional re-plans from the lengths in device memory at every replay
    lens_a, lens_b = [3000, 700, 1500], [100, 0, 5800]
    inp = workloads.mla_inputs(B=3, q_len=1, H=64, seq_lens=lens_a, pool_rows=6000, seed=73, device=DEV)
    inp_b = workloads.mla_inputs(B=3, q_len=1, H=64, seq_lens=lens_b, pool_rows=6000, seed=74,
                                 device=DEV)
    idx = torch.zeros((6000,), dtype=torch.int32, device=DEV)
    idx[:inp.kv_indices.numel()] = inp.kv_indices
    p = g.mla_problem(inp.q_lat, inp.q_pe, inp.pool, idx, inp.kv_indptr, inp.seq_lens,
                      batch=3, q_len=1, num_heads=64, max_num_keys=6000, scale=inp.scale,
                      kv_scale=inp.kv_scale, d_v=512)
    ws = torch.empty((g.decode_proportional_workspace_bytes(p, 4) // 4 + 64,), dtype=torch.float32,
                     device=DEV)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out, lse = run_prop(p, 512, 4, 0, 32, stream=s, ws=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g.decode_proportional(p, out, lse, np=4, cap=0, block_k=32, workspace=ws, stream=s)
    idx_b = torch.zeros_like(idx)
    idx_b[:inp_b.kv_indices.numel()] = inp_b.kv_indices
    data = {False: (inp.q_lat.clone(), inp.q_pe.clone(), inp.pool.clone(), idx.clone(),
                    inp.kv_indptr.clone(), inp.seq_lens.clone()),
            True: (inp_b.q_lat, inp_b.q_pe, inp_b.pool, idx_b, inp_b.kv_indptr, inp_b.seq_lens)}
    refs = {False: oracle_mla(inp), True: oracle_mla(inp_b)}
    for new in (True, False, True):
        log("proportional graph replay, lengths %s" % (lens_b if new else lens_a))
        for dst, src in zip((inp.q_lat, inp.q_pe, inp.pool, idx, inp.kv_indptr, inp.seq_lens),
                            data[new]):
            dst.copy_(src)
        out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = refs[new]
        compare(out, lse, ref_o, ref_l, "proportional graph replay %s" % (lens_b if new else lens_a))


def test_skewed_batch_full_size_sampled():
    # one request of 131072 keys among 31 of 2048, in the launch the benchmark times
    from gpu_util import sample_rows
    inp = workloads.mla_skewed(DEV)
    torch.cuda.synchronize()
    p = mla_problem(inp)
    np_, bk = g.decode_plan(p)
    log("skewed batch proportional np=%d bk=%d" % (np_, bk))
    out, lse = run_prop(p, 512, np_, 0, bk)
    torch.cuda.synchronize()
    rows = sample_rows(inp.B, 1, inp.H, 24, seed=7) + list(range(0, 64, 9))
    rows = sorted(set(rows))
    ref_o, ref_l = oracle_mla(inp, rows)
    compare(out[rows], lse[rows], ref_o, ref_l, "skewed batch proportional")


@pytest.mark.parametrize("kind", ["mla", "gqa"])
def test_proportional_with_planner_choices(kind):
    # np = 0 and block_k = 0: the wave-aligned planner's budget and the tile rule, as decode
    lens = [5000, 17, 0, 1200, 64]
    if kind == "mla":
        inp = workloads.mla_inputs(B=5, q_len=1, H=64, seq_lens=lens, pool_rows=6400, seed=83,
                                   device=DEV)
        p, d_v, ref = mla_problem(inp), 512, oracle_mla
    else:
        inp = workloads.gqa_inputs(B=5, Hq=32, Hkv=4, D=128, page_size=16, seq_lens=lens,
                                   num_pages=420, q_len=1, seed=93, device=DEV)
        p, d_v, ref = gqa_problem(inp), 128, oracle_gqa
    torch.cuda.synchronize()
    log("proportional %s with planner choices np=%d bk=%d" % ((kind,) + tuple(g.decode_plan(p))))
    out, lse = run_prop(p, d_v)
    torch.cuda.synchronize()
    ref_o, ref_l = ref(inp)
    compare(out, lse, ref_o, ref_l, "proportional %s planner choices" % kind)


def test_sparse_proportional_many_queries():
    # 100 queries: the slot lookup in the MLA kernel walks the prefix table 64 requests at a time
    inp = workloads.sparse_mla_inputs(num_queries=100, topk=256, cache_rows=8192, seed=4700,
                                      invalid_frac=0.05, all_invalid=(70,), device=DEV)
    torch.cuda.synchronize()
    log("sparse proportional 100 queries")
    out, lse = run_prop(mla_problem(inp), 448, 2, 0, 32)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "sparse proportional 100 queries")
    assert torch.all(lse[70 * 64:71 * 64] == -float("inf"))
