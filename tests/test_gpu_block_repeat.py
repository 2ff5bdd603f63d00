"""gemm_block_repeat (Warp issue #1965 "Spike" workload) against the oracle:
C = repeats * Q(A[:, :TK]) @ Q(B[:TK, :]) on a 2048 x 2048 output, every tile
variant and both 16-bit types; bit-exact on small-integer inputs.  Both arms
of the issue's comparison: the register accumulator with swizzled LDS
(gemm_block_repeat) and the shared-memory API (gemm_block_repeat_lds_api:
plain LDS tiles, C read and written through LDS on every repeat)."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from mma_fragment_layouts_amd import inputs
from oracle import reference as R

from _gpu import DT, device, host, q16, say, stream

pytestmark = pytest.mark.gpu

VARIANTS = [(64, 64, 64, 64), (64, 64, 64, 128), (64, 64, 64, 256), (32, 32, 32, 128), (128, 128, 32, 128),
            (128, 128, 32, 256)]
APIS = {"register": mfl.gemm_block_repeat, "lds": mfl.gemm_block_repeat_lds_api}


@pytest.mark.parametrize("api", sorted(APIS))
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("tm,tn,tk,threads", VARIANTS)
def test_block_repeat(tm, tn, tk, threads, fmt, api):
    a, bt = inputs.block_repeat(tm, tn, tk)
    say("block repeat", api, tm, tn, tk, threads, fmt)
    c = torch.full((2048, 2048), np.nan, device=device())
    APIS[api](DT[fmt], tm, tn, tk, threads, 64, 2048, 2048, q16(a, fmt), q16(bt, fmt), c, stream())
    ch = host(c)
    assert not np.isnan(ch).any()
    assert R.rel_error(ch, R.block_repeat_ref(a, bt, tk, 64, fmt)) <= 1e-5


@pytest.mark.parametrize("api", sorted(APIS))
@pytest.mark.parametrize("tm,tn,tk,threads", VARIANTS)
def test_block_repeat_integer_exact(tm, tn, tk, threads, api):
    rng = np.random.default_rng(tm + tk + threads)
    a = rng.integers(-4, 5, (512, tk)).astype(np.float32)
    bt = rng.integers(-4, 5, (256, tk)).astype(np.float32)
    say("block repeat exact", api, tm, tn, tk, threads)
    c = torch.empty((512, 256), device=device())
    APIS[api](mfl.BF16, tm, tn, tk, threads, 7, 512, 256, q16(a, "bf16"), q16(bt, "bf16"), c, stream())
    assert np.array_equal(host(c), 7 * (a.astype(np.int64) @ bt.T.astype(np.int64)).astype(np.float32))


@pytest.mark.parametrize("api", sorted(APIS))
def test_zero_repeats_gives_zero(api):
    a, bt = inputs.block_repeat(64, 64, 64, 256, 256)
    c = torch.full((256, 256), 5.0, device=device())
    say("block repeat zero", api)
    APIS[api](mfl.F16, 64, 64, 64, 256, 0, 256, 256, q16(a, "f16"), q16(bt, "f16"), c, stream())
    assert np.all(host(c) == 0)
