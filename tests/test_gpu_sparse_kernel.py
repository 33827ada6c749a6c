"""GPU parity of the split kernel that serves 512-byte fp8 rows of one cache (the sparse top-k
layout: 448 latent and 64 rope elements per row; its score waves each cover all 64 query rows of
a CTA), against the fp64 CPU oracle, beyond the shapes the general parity tests run on it: wide
dynamic range, head counts that leave row blocks partly empty, draft windows, the
allocation-free entry point and determinism.

Bars: those of gpu_util (the project bar) on the fp32 result and on decode()'s bf16 output after
half a bf16 ulp of the reference value, as in test_gpu_numerics.
"""
import numpy as np
import pytest
import torch

import gqa_plan_splits_amd as g
import workloads
from gpu_util import compare, log, mla_problem, oracle_mla, run_decode
from test_gpu_numerics import CASES, compare_bf16_output

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"
DQK, DV = 512, 448


def rows512(B, q_len, H, lens, seed, pool_rows=None):
    return workloads.mla_inputs(B=B, q_len=q_len, H=H, seq_lens=lens,
                                pool_rows=pool_rows or sum(lens) + 100, d_qk=DQK, d_v=DV,
                                seed=seed, device=DEV, fused_q=True)


def fp32_result(p, np_, bk):
    rows = p.rows
    po = torch.empty((rows, np_, DV), dtype=torch.float32, device=DEV)
    pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
    g.decode_split(p, np_, bk, po, pl)
    if np_ == 1:
        return po[:, 0], pl[:, 0]
    out = torch.empty((rows, DV), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce_f32(rows, np_, DV, po, pl, out, lse)
    return out, lse


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("q_len", [1, 4])
def test_sparse_rows_wide_dynamic_range(case, q_len):
    inp = CASES[case](rows512(3, q_len, 64, [2500, 700, 3], seed=201 + q_len, pool_rows=4000))
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp)
    planner_np, planner_bk = g.decode_plan(p)
    for np_, bk in ((1, 64), (planner_np, planner_bk)):
        what = "512-byte rows %s q_len=%d np=%d bk=%d" % (case, q_len, np_, bk)
        log(what)
        o32, l32 = fp32_result(p, np_, bk)
        torch.cuda.synchronize()
        compare(o32, l32, ref_o, ref_l, what + " fp32")
        out, lse = run_decode(p, DV, np_, bk)
        torch.cuda.synchronize()
        compare_bf16_output(out, lse, ref_o, ref_l, what + " bf16")


@pytest.mark.parametrize("H,q_len", [(16, 1), (40, 1), (128, 1), (16, 3), (24, 4)])
@pytest.mark.parametrize("np_,bk", [(1, 64), (5, 32), (0, 0)])
def test_sparse_rows_head_counts(H, q_len, np_, bk):
    # rows per request q_len * H: fewer than 64 (one row block partly empty), more than 64 (two
    # row blocks), and draft positions that straddle row blocks
    inp = rows512(4, q_len, H, [900, 64, 1, 2000], seed=211 + H + q_len)
    torch.cuda.synchronize()
    log("512-byte rows H=%d q_len=%d np=%d bk=%d" % (H, q_len, np_, bk))
    out, lse = run_decode(mla_problem(inp), DV, np_, bk)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle_mla(inp)
    compare(out, lse, ref_o, ref_l, "512-byte rows H=%d q_len=%d np=%d" % (H, q_len, np_))


def test_sparse_rows_scratch_invariance_and_determinism():
    inp = workloads.sparse_mla_inputs(num_queries=40, topk=1500, cache_rows=30000, seed=231,
                                      invalid_frac=0.1, device=DEV)
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp, n_threads=8)
    base_o, base_l = run_decode(p, DV, 1, 64)
    torch.cuda.synchronize()
    compare(base_o, base_l, ref_o, ref_l, "512-byte rows np=1")
    for np_, bk in [(3, 32), (8, 64), (0, 0)]:
        log("512-byte rows invariance np=%d bk=%d" % (np_, bk))
        o, l = run_decode(p, DV, np_, bk)
        torch.cuda.synchronize()
        compare(o, l, ref_o, ref_l, "512-byte rows np=%d" % np_)
        assert (o.float() - base_o.float()).abs().max().item() <= 4e-3
        fin = torch.isfinite(base_l)
        assert torch.equal(fin, torch.isfinite(l))
        assert ((l[fin] - base_l[fin]).abs() / base_l[fin].abs().clamp(min=1)).max().item() <= 1e-5
    o1, l1 = run_decode(p, DV, 8, 32)
    out = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    g.decode_scratch(p, out, lse, np=8, block_k=32)
    o2, l2 = run_decode(p, DV, 8, 32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, out) and torch.equal(l1, lse)
    assert np.isfinite(ref_l).any()
