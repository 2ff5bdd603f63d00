"""attention_split_fp32 against the oracle: fp64 softmax(Q Q16(K)^T) Q16(V)
with Q at its original values; normwise error <= 5e-6.  Both device
algorithms (materialised scores, fused online softmax) and both chain counts;
small sizes in full, the 2048 x 32768 x 128 workload on sampled query rows."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from mma_fragment_layouts_amd import inputs
from oracle import reference as R

from _gpu import dev32, device, host, say, stream

pytestmark = pytest.mark.gpu
ALGOS = [mfl.ATTN_MATERIALISED, mfl.ATTN_FUSED]


def run_attention(q, k, v, chains, algo):
    nq, d = q.shape
    nk = k.shape[0]
    ws_bytes = mfl.attention_workspace_bytes(nq, nk, d, algo)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=device())
    o = torch.full((nq, d), np.nan, device=device())
    mfl.attention_split_fp32(nq, nk, d, dev32(q), dev32(k), dev32(v), chains, algo, o, ws, ws_bytes, stream())
    return host(o)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("chains", [1, 2])
# key chunks of 64 per workgroup slice: 1, 3, 5, 1, 2 and 4 (odd counts take the
# fused kernel's odd tail); (384, 4096) maps workgroups to XCDs by slice
@pytest.mark.parametrize("nq,nk", [(128, 128), (128, 384), (256, 640), (256, 1024), (384, 4096), (128, 8192)])
def test_attention_small(nq, nk, chains, algo):
    q, k, v = inputs.attention(nq, nk)
    say("attention", nq, nk, chains, algo)
    o = run_attention(q, k, v, chains, algo)
    err = R.rel_error(o, R.attention_ref(q, k, v))
    print(f"attention {nq}x{nk} chains={chains} algo={algo} err={err:.3e}")
    assert err <= 5e-6


@pytest.mark.parametrize("algo", ALGOS)
def test_attention_uniform_closed_form(algo):
    """Q = 0: every score is 0, P is uniform and O is the column mean of Q16(V)."""
    _, k, v = inputs.attention(128, 2048)
    q = np.zeros((128, 128), np.float32)
    say("attention Q=0", algo)
    o = run_attention(q, k, v, 2, algo)
    assert R.rel_error(o, R.attention_ref(q, k, v)) <= 5e-6


@pytest.mark.parametrize("algo", ALGOS)
def test_attention_large_scores(algo):
    """Scores of order 10 (Q scaled by 100): the running max moves between key
    chunks and slices, exercising the rescaling of the fused kernel."""
    q, k, v = inputs.attention(256, 4096)
    q = (q * 100.0).astype(np.float32)
    say("attention large scores", algo)
    o = run_attention(q, k, v, 2, algo)
    assert R.rel_error(o, R.attention_ref(q, k, v)) <= 5e-6


def test_attention_full_size_sampled():
    q, k, v = inputs.attention()
    errs = {}
    rows = np.random.default_rng(15).choice(2048, 64, replace=False)
    ref = R.attention_ref(q[rows], k, v)
    for algo in ALGOS:
        for chains in (1, 2):
            say("attention 2048x32768", chains, algo)
            o = run_attention(q, k, v, chains, algo)
            assert not np.isnan(o).any()
            errs[(algo, chains)] = R.rel_error(o[rows], ref)
    print("attention full-size errors (algo, chains):", errs)
    assert errs[(mfl.ATTN_MATERIALISED, 2)] <= 5e-6
    assert errs[(mfl.ATTN_FUSED, 2)] <= 5e-6


# ---- algo 2: K and V split as well; reference on the original fp32 K and V

@pytest.mark.parametrize("chains", [1, 2])
@pytest.mark.parametrize("nq,nk", [(128, 128), (128, 384), (256, 640), (384, 4096)])
def test_attention_split_kv_small(nq, nk, chains):
    q, k, v = inputs.attention(nq, nk)
    say("attention split kv", nq, nk, chains)
    o = run_attention(q, k, v, chains, mfl.ATTN_FUSED_SPLIT_KV)
    err = R.rel_error(o, R.attention_ref(q, k, v, round_kv=False))
    print(f"attention split-kv {nq}x{nk} chains={chains} err={err:.3e}")
    assert err <= 5e-6


def test_attention_split_kv_large_scores():
    q, k, v = inputs.attention(256, 4096)
    q = (q * 100.0).astype(np.float32)
    say("attention split kv large scores")
    o = run_attention(q, k, v, 2, mfl.ATTN_FUSED_SPLIT_KV)
    assert R.rel_error(o, R.attention_ref(q, k, v, round_kv=False)) <= 5e-6


def test_attention_split_kv_full_size_removes_the_rounding_floor():
    """2048 x 32768: against the reference on the ORIGINAL K and V, rounding K
    and V once (algo 1) leaves an error floor; splitting them (algo 2) removes it."""
    q, k, v = inputs.attention()
    rows = np.random.default_rng(16).choice(2048, 64, replace=False)
    ref = R.attention_ref(q[rows], k, v, round_kv=False)
    errs = {}
    for algo in (mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV):
        say("attention vs fp32 K/V reference", algo)
        o = run_attention(q, k, v, 2, algo)
        assert not np.isnan(o).any()
        errs[algo] = R.rel_error(o[rows], ref)
    print("errors against the fp32-K/V reference (algo 1, algo 2):", errs)
    assert errs[mfl.ATTN_FUSED_SPLIT_KV] <= 5e-6
    assert errs[mfl.ATTN_FUSED] >= 10 * errs[mfl.ATTN_FUSED_SPLIT_KV]
