"""The diagnostic read kernel behind bench.py's read ceiling: it reads every element once
(the partial sums of ones add up to the count, including a ragged tail) and rejects bad
arguments."""
import numpy as np
import pytest

import top_select_gumbel_amd as ts
from gpu_helpers import banner, torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [1, 3, 8192, 1_000_003, 64 * 151936])
def test_read_ceiling_reads_every_element(n):
    torch = torch_cuda()
    banner(f"read ceiling n={n}")
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    out = ts.ts_read_ceiling(x)
    torch.cuda.synchronize()
    assert out.numel() == ts.read_ceiling_partials(n)
    assert float(out.double().sum().item()) == float(n)   # integer partials are exact


def test_read_ceiling_rejects_misaligned_pointer():
    torch = torch_cuda()
    banner("read ceiling misaligned")
    lib = ts.load_library()
    x = torch.ones(64, dtype=torch.float32, device="cuda:0")
    out = torch.zeros(4, dtype=torch.float32, device="cuda:0")
    rc = lib.ts_read_ceiling(x.data_ptr() + 4, 16, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == ts.TS_ERR_INVALID_ARG
    rc = lib.ts_read_ceiling(x.data_ptr(), -1, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == ts.TS_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert float(out.abs().sum().item()) == 0.0
