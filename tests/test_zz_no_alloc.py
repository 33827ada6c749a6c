"""decode_scratch (the allocation-free decode) against decode() through the C ABI."""
import pytest
import torch

import gqa_plan_splits_amd as g
import workloads
from gpu_util import gqa_problem, log, mla_problem, run_decode

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


def scratch_decode(problem, d_v, np_, bk):
    out = torch.empty((problem.rows, d_v), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((problem.rows,), dtype=torch.float32, device=DEV)
    g.decode_scratch(problem, out, lse, np=np_, block_k=bk)
    return out, lse


def test_decode_scratch_matches_decode_on_two_calls():
    # two calls in a row, the second smaller: the scratch array keeps the first call's partials,
    # which the second must neither need nor see
    big = workloads.mla_inputs(B=4, q_len=1, H=64, seq_lens=[20000, 20000, 9000, 333],
                               pool_rows=49333, seed=141, device=DEV)
    small = workloads.mla_inputs(B=2, q_len=2, H=32, seq_lens=[3000, 100], pool_rows=3100,
                                 seed=142, device=DEV)
    torch.cuda.synchronize()
    for name, inp, np_, bk in (("big", big, 0, 0), ("small", small, 4, 64)):
        p = mla_problem(inp)
        log("decode_scratch %s np=%d" % (name, np_))
        ref_o, ref_l = run_decode(p, 512, np_, bk)
        out, lse = scratch_decode(p, 512, np_, bk)
        torch.cuda.synchronize()
        # the same plan and kernels: bit-identical to decode()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), name


def test_decode_scratch_gqa_and_np1():
    lens = [700, 33, 1, 0, 1600, 16]
    inp = workloads.gqa_inputs(B=6, Hq=16, Hkv=2, D=128, page_size=16, seq_lens=lens, num_pages=300,
                               seed=143, device=DEV)
    torch.cuda.synchronize()
    p = gqa_problem(inp)
    for np_, bk in ((8, 32), (1, 64)):
        ref_o, ref_l = run_decode(p, 128, np_, bk)
        out, lse = scratch_decode(p, 128, np_, bk)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), np_


def test_decode_scratch_rejects_partials_beyond_the_array():
    # 4096 rows x 256 partitions x 512 fp32 values is 2 GiB of partials
    inp = workloads.mla_inputs(B=64, q_len=1, H=64, seq_lens=[300] * 64, pool_rows=19200, seed=144,
                               device=DEV)
    torch.cuda.synchronize()
    p = mla_problem(inp)
    with pytest.raises(g.GqaError) as e:
        scratch_decode(p, 512, 256, 32)
    assert e.value.status == -3 and "static scratch holds" in str(e.value)
