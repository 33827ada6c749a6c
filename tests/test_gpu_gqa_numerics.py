"""GPU parity of the GQA split kernels (the kv-head-pair kernel, the one-head kernel with one and
two 16-row waves, and the kernel of two 32-row waves) at wider dynamic range than N(0,1) data,
against the fp64 CPU oracle.

The kernels multiply bf16 queries by bf16 keys (exact products, fp32 sums), keep an fp32
running maximum and sum, and hand the weights 2^(score - max) to the PV MFMA rounded to bf16,
so each weight carries a relative error of at most 2^-9 and the output at most
2^-9 * max|v - o| beyond fp32 rounding; the log-sum-exp comes from the fp32 sums.  The cases:
queries x4 and x16 (scores spread over many octaves within and across 16-token tiles, and
nearly one-hot rows), one dominant key per tile, and values x4 (outputs up to about 16).

Bars: those of gpu_util (the project bar) on the fp32 result, and on decode()'s bf16 output
after half a bf16 ulp of the reference value, as for the MLA kernels.
"""
import pytest
import torch

import gqa_plan_splits_amd as g
import workloads
from gpu_util import compare, gqa_problem, log, oracle_gqa, run_decode
from test_gpu_numerics import compare_bf16_output

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"

CASES = {
    "q_x4": lambda inp: workloads.gqa_scaled(inp, q_mul=4.0),
    "q_x16": lambda inp: workloads.gqa_scaled(inp, q_mul=16.0),
    "dominant_key_per_tile": lambda inp: workloads.gqa_dominant_keys(inp, mul=8.0, seed=5),
    "q_x4_v_x4": lambda inp: workloads.gqa_scaled(inp, q_mul=4.0, v_mul=4.0),
    "dominant_key_v_x4": lambda inp: workloads.gqa_scaled(workloads.gqa_dominant_keys(inp, mul=8.0, seed=6),
                                                          v_mul=4.0),
}

# (Hq, Hkv, q_len): kv-head pairs (group 8), one-head CTAs of one 16-row wave (3 kv heads), two
# 16-row waves (24 rows) and two 32-row waves (64 rows on one kv head)
SHAPES = [(64, 8, 1), (12, 3, 1), (24, 1, 1), (64, 1, 1)]


def fp32_result(p, np_, bk):
    rows = p.rows
    po = torch.empty((rows, np_, 128), dtype=torch.float32, device=DEV)
    pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
    g.decode_split(p, np_, bk, po, pl)
    if np_ == 1:
        return po[:, 0], pl[:, 0]
    out = torch.empty((rows, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce_f32(rows, np_, 128, po, pl, out, lse)
    return out, lse


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("Hq,Hkv,q_len", SHAPES)
def test_gqa_wide_dynamic_range(case, Hq, Hkv, q_len):
    lens = [1500, 40, 700, 3]
    inp = workloads.gqa_inputs(B=4, Hq=Hq, Hkv=Hkv, D=128, page_size=16, seq_lens=lens,
                               num_pages=200, q_len=q_len, seed=61, device=DEV)
    inp = CASES[case](inp)
    torch.cuda.synchronize()
    p = gqa_problem(inp)
    ref_o, ref_l = oracle_gqa(inp)
    planner_np, planner_bk = g.decode_plan(p)
    for np_, bk in ((1, 32), (planner_np, planner_bk)):
        what = "gqa %s Hq=%d Hkv=%d np=%d" % (case, Hq, Hkv, np_)
        log(what)
        o32, l32 = fp32_result(p, np_, bk)
        torch.cuda.synchronize()
        compare(o32, l32, ref_o, ref_l, what + " fp32")
        out, lse = run_decode(p, 128, np_, bk)
        torch.cuda.synchronize()
        compare_bf16_output(out, lse, ref_o, ref_l, what + " bf16")
