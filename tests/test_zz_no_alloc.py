"""attention_split_fp32_static, the entry point that allocates nothing: the
same kernels as attention_split_fp32 with the workspace in a static device
array of MFL_ATTN_STATIC_SCRATCH_BYTES per GPU.  Checked through the C ABI
against the workspace entry point (bit for bit: same kernels, same operands)
and the oracle, on two calls in a row, the second with a smaller input (the
array keeps the first call's contents, which must not leak into the second);
sizes beyond the array are refused before any device work."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from mma_fragment_layouts_amd import inputs
from oracle import reference as R

from _gpu import dev32, device, host, say, stream

pytestmark = pytest.mark.gpu


def with_workspace(q, k, v, chains, algo):
    nq, d = q.shape
    nk = k.shape[0]
    wsb = mfl.attention_workspace_bytes(nq, nk, d, algo)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device())
    o = torch.full((nq, d), np.nan, device=device())
    mfl.attention_split_fp32(nq, nk, d, dev32(q), dev32(k), dev32(v), chains, algo, o, ws, wsb, stream())
    return host(o)


def static(q, k, v, chains, algo):
    nq, d = q.shape
    nk = k.shape[0]
    o = torch.full((nq, d), np.nan, device=device())
    mfl.attention_split_fp32_static(nq, nk, d, dev32(q), dev32(k), dev32(v), chains, algo, o, stream())
    return host(o)


# (first call, second smaller call) per algorithm; the first fills most of the
# static array where the algorithm allows it
SIZES = {mfl.ATTN_MATERIALISED: ((256, 8192), (128, 1024)),
         mfl.ATTN_FUSED: ((2048, 32768), (256, 4096)),
         mfl.ATTN_FUSED_SPLIT_KV: ((2048, 32768), (128, 640))}


@pytest.mark.parametrize("chains", [1, 2])
@pytest.mark.parametrize("algo", [mfl.ATTN_MATERIALISED, mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV])
def test_static_matches_workspace_entry_on_two_calls(algo, chains):
    for nq, nk in SIZES[algo]:
        assert mfl.attention_workspace_bytes(nq, nk, 128, algo) <= mfl.ATTN_STATIC_SCRATCH_BYTES
        q, k, v = inputs.attention(nq, nk)
        say("no-alloc attention", algo, chains, nq, nk)
        got = static(q, k, v, chains, algo)
        want = with_workspace(q, k, v, chains, algo)
        assert not np.isnan(got).any()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (nq, nk)
        ref = R.attention_ref(q, k, v, round_kv=algo != mfl.ATTN_FUSED_SPLIT_KV)
        assert R.rel_error(got, ref) <= 5e-6, (nq, nk)


def test_static_refuses_sizes_beyond_the_array():
    """The materialised scores of 2048 x 32768 need 256 MiB: refused with
    MFL_ESCRATCH before any device work, the output left as it was."""
    nq, nk = 2048, 32768
    assert mfl.attention_workspace_bytes(nq, nk, 128, mfl.ATTN_MATERIALISED) > mfl.ATTN_STATIC_SCRATCH_BYTES
    q = torch.zeros((nq, 128), device=device())
    k = torch.zeros((nk, 128), device=device())
    o = torch.full((nq, 128), 7.0, device=device())
    with pytest.raises(mfl.MflError) as e:
        mfl.attention_split_fp32_static(nq, nk, 128, q, k, k, 2, mfl.ATTN_MATERIALISED, o, stream())
    assert e.value.status == mfl.ESCRATCH
    assert np.all(host(o) == 7.0)
