"""The benchmark's data-movement ceiling kernels run through the C ABI (they move bytes into LDS
and discard them: there is no output to compare, only the launch and its completion)."""
import pytest
import torch

import gqa_plan_splits_amd as g

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def test_stream_read_runs():
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    g.bw_stream_read(buf, buf.numel(), 256)
    torch.cuda.synchronize()


@pytest.mark.parametrize("whole", [False, True])
@pytest.mark.parametrize("row_bytes", [576, 512])
def test_gather_rows_runs(row_bytes, whole):
    pool = torch.zeros((100000, row_bytes), dtype=torch.uint8, device="cuda")
    idx = torch.randperm(100000, device="cuda")[:64 * 1000].to(torch.int32)
    torch.cuda.synchronize()
    (g.bw_gather_whole_rows if whole else g.bw_gather_rows)(pool, row_bytes, idx, idx.numel(), 256)
    torch.cuda.synchronize()
