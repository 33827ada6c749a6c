"""GPU parity of the MLA split kernel at wide dynamic range, against the fp64 CPU oracle.

The kernel multiplies the bf16 query by the stored fp8 K decoded exactly to bf16 (exact
products, fp32 sums), stores the softmax weights 2^(score - m + 8) relative to an integer
running maximum m as fp16, and multiplies them by V decoded exactly to fp16 (fp32 sums); the
output is normalized by the sum of the stored weights and the LSE comes from the exact ones.
The cases drive the regimes where rounding could show: scores spread over tens of octaves
within and across tiles, query rows whose elements span 20 octaves, pool bytes at the largest
e4m3 magnitudes and in the subnormal range, and one dominant key per tile.

Bars (the oracle is unsplit fp64 softmax attention over the same stored bytes, the comparison
the moonmath-amd README's "Numerics" paragraph describes: an fp32-or-better reference over the
same dequantized KV):
  * the fp32 result (decode_split, then splitk_reduce_f32 when np > 1): the project bar,
    max|dO| <= 1e-2, max|dO| / max|O_ref| <= 1e-2, |d lse2| <= 1e-4 max(1, |lse2|);
  * the bf16 output of decode(): the same bars after allowing the output's own rounding, half a
    bf16 ulp of the reference value (with values up to 448/32 = 14 that half ulp is 2^-5, above
    the 1e-2 absolute bar by itself).
"""
import numpy as np
import pytest
import torch

import gqa_plan_splits_amd as g
import workloads
from gpu_util import LSE_RTOL, OUT_ATOL, OUT_REL, compare, log, mla_problem, oracle_mla, run_decode

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"

CASES = {
    "q_x8": lambda inp: workloads.scaled_queries(inp, 8.0),
    "q_x32": lambda inp: workloads.scaled_queries(inp, 32.0),
    "q_rows_2^-20_to_1": lambda inp: workloads.wide_range_queries(inp, 20.0, 1.0, seed=11),
    "q_rows_2^-20_to_32_extreme_pool": lambda inp: workloads.extreme_pool(
        workloads.wide_range_queries(inp, 20.0, 32.0, seed=12), seed=13),
    "extreme_pool": lambda inp: workloads.extreme_pool(inp, frac_large=0.15, frac_subnormal=0.15, seed=14),
    "q_x8_extreme_pool": lambda inp: workloads.extreme_pool(workloads.scaled_queries(inp, 8.0), seed=15),
    "dominant_key_per_tile": lambda inp: workloads.dominant_keys(inp, seed=16),
}


def base_input(q_len):
    # three ragged requests: several tiles, a short one, one shorter than the draft window
    return workloads.mla_inputs(B=3, q_len=q_len, H=64, seq_lens=[2500, 700, 3], pool_rows=4000,
                                seed=101 + q_len, device=DEV)


def fp32_result(p, np_, bk):
    """decode_split, then (np > 1) the fp32 merge: the kernel's arithmetic before bf16 rounding."""
    rows = p.rows
    po = torch.empty((rows, np_, 512), dtype=torch.float32, device=DEV)
    pl = torch.empty((rows, np_), dtype=torch.float32, device=DEV)
    g.decode_split(p, np_, bk, po, pl)
    if np_ == 1:
        return po[:, 0], pl[:, 0]
    out = torch.empty((rows, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((rows,), dtype=torch.float32, device=DEV)
    g.splitk_reduce_f32(rows, np_, 512, po, pl, out, lse)
    return out, lse


def half_ulp_bf16(x):
    """Half a bf16 ulp at |x| (8 significant bits): 2^(floor(log2 |x|) - 8); 0 at 0."""
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.exp2(e - 8), 0.0)


def compare_bf16_output(out, lse, ref_o, ref_l, what):
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.isfinite(o)), what + ": non-finite output"
    empty = ~np.isfinite(ref_l)
    assert np.array_equal(empty, ~np.isfinite(l)) and np.all(o[empty] == 0), what + ": empty rows"
    excess = np.abs(o - ref_o) - half_ulp_bf16(ref_o)
    worst = float(excess.max())
    scale = float(np.abs(ref_o).max())
    assert worst <= OUT_ATOL, "%s: max(|dO| - half ulp) %.3g > %g" % (what, worst, OUT_ATOL)
    assert worst <= OUT_REL * scale, "%s: relative %.3g > %g" % (what, worst / scale, OUT_REL)
    lerr = np.abs(l[~empty] - ref_l[~empty]) / np.maximum(1.0, np.abs(ref_l[~empty]))
    assert float(lerr.max()) <= LSE_RTOL, "%s: lse2 error %.3g" % (what, float(lerr.max()))
    return worst


@pytest.mark.parametrize("case", list(CASES))
@pytest.mark.parametrize("q_len", [1, 4])
def test_mla_wide_dynamic_range_matches_oracle(case, q_len):
    inp = CASES[case](base_input(q_len))
    torch.cuda.synchronize()
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp)
    planner_np, planner_bk = g.decode_plan(p)
    for np_, bk in ((1, 64), (planner_np, planner_bk)):
        what = "%s q_len=%d np=%d bk=%d" % (case, q_len, np_, bk)
        log("numerics " + what)
        o32, l32 = fp32_result(p, np_, bk)
        torch.cuda.synchronize()
        max_abs, rel, lse_err = compare(o32, l32, ref_o, ref_l, what + " fp32")
        out, lse = run_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        excess = compare_bf16_output(out, lse, ref_o, ref_l, what + " bf16")
        log("  fp32: max|dO| %.3g rel %.3g lse2 %.3g; bf16: max(|dO| - half ulp) %.3g; max|O| %.3g, "
            "lse2 %.1f..%.1f" % (max_abs, rel, lse_err, excess, float(np.abs(ref_o).max()),
                                 float(np.min(ref_l[np.isfinite(ref_l)])), float(np.max(ref_l))))


@pytest.mark.parametrize("how", ["request", "contiguous"])
def test_mla_sorted_and_contiguous_slot_lists_match_oracle(how):
    # slot lists in pool order (sorted per request) and a plain arange: any order of a request's
    # keys is legal and gives the same attention (the moonmath-amd README's MLA decode example
    # uses contiguous slots).  Inputs are built on the stream the kernels run on (the default
    # stream) and synchronized before the first launch.
    lens = [20000, 20000, 9000, 333]
    inp = workloads.mla_inputs(B=4, q_len=1, H=64, seq_lens=lens, pool_rows=sum(lens), seed=131,
                               device=DEV)
    inp = workloads.sorted_slots(inp, how)
    torch.cuda.synchronize()
    idx = inp.kv_indices.cpu()
    assert int(idx.min()) >= 0 and int(idx.max()) < inp.pool.shape[0]
    p = mla_problem(inp)
    ref_o, ref_l = oracle_mla(inp, n_threads=8)
    planner_np, planner_bk = g.decode_plan(p)
    for np_, bk in ((1, 64), (planner_np, planner_bk), (16, 32)):
        log("sorted slots %s np=%d bk=%d" % (how, np_, bk))
        out, lse = run_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        compare(out, lse, ref_o, ref_l, "slots %s np=%d" % (how, np_))
