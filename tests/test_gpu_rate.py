"""mfma_rate_probe, the MFMA-rate microbenchmark behind the benchmark's
measured ceiling: with unit operands every thread's sum has a closed form
(16 chains started at 0..15, each adding K = 32 unit products per round, four
accumulator values per chain); with hashed operands the result is finite and
the same on every call."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl

from _gpu import device, host, say, stream

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [mfl.F16, mfl.BF16])
@pytest.mark.parametrize("iters", [0, 1, 37, 4096])
def test_rate_probe_unit_operands(dtype, iters):
    out = torch.full((mfl.RATE_PROBE_OUTPUTS,), np.nan, device=device())
    say("rate probe", dtype, iters)
    mfl.mfma_rate_probe(dtype, iters, 0, out, stream())
    want = 4 * sum(range(16)) + 16 * 4 * 32 * iters      # = 480 + 2048 * iters
    assert np.all(host(out) == np.float32(want))


@pytest.mark.parametrize("dtype", [mfl.F16, mfl.BF16])
def test_rate_probe_hashed_operands_repeatable(dtype):
    a = torch.empty((mfl.RATE_PROBE_OUTPUTS,), device=device())
    b = torch.empty_like(a)
    say("rate probe hashed", dtype)
    mfl.mfma_rate_probe(dtype, 64, 12345, a, stream())
    mfl.mfma_rate_probe(dtype, 64, 12345, b, stream())
    ha, hb = host(a), host(b)
    assert np.all(np.isfinite(ha))
    assert np.array_equal(ha.view(np.uint32), hb.view(np.uint32))
    # values in [1, 2): each of the 16 x 4 accumulator values grows by 32..128 per round
    assert np.all(ha >= 480 + 64 * 64 * 32) and np.all(ha <= 480 + 64 * 64 * 128)


def test_rate_probe_rejects_bad_arguments():
    out = torch.empty((mfl.RATE_PROBE_OUTPUTS,), device=device())
    with pytest.raises(mfl.MflError):
        mfl.mfma_rate_probe(7, 1, 0, out, stream())
    with pytest.raises(mfl.MflError):
        mfl.mfma_rate_probe(mfl.F16, -1, 0, out, stream())
