"""attention_split_fp32 against the oracle: fp64 softmax(Q Q16(K)^T) Q16(V)
with Q at its original values; normwise error <= 5e-6.  Both device
algorithms (materialised scores, fused online softmax) and both chain counts;
every output row at every size, including 2048 queries at 8,192, 32,768
and 131,072 keys."""
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


@pytest.mark.parametrize("chains", [1, 2])
def test_attention_materialised_uneven_slices(chains):
    """128 queries x 32,896 keys: 514 chunks of 64 keys, so the materialised
    path's key slices hold 3 chunks each and the last one a single chunk.
    Every row against the oracle."""
    q, k, v = inputs.attention(128, 514 * 64)
    say("attention uneven slices", chains)
    o = run_attention(q, k, v, chains, mfl.ATTN_MATERIALISED)
    err = R.rel_error(o, R.attention_ref(q, k, v))
    print(f"attention 128x{514 * 64} chains={chains} materialised err={err:.3e}")
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


def _all_rows(nk, algos=ALGOS, chains_list=(1, 2)):
    """Every query row of 2048 x nk x 128 through each algorithm and chain
    count, against the oracle; returns {(algo, chains): error}."""
    q, k, v = inputs.attention(2048, nk)
    ref = R.attention_ref(q, k, v)
    errs = {}
    for algo in algos:
        for chains in chains_list:
            say("attention 2048 x", nk, "chains", chains, "algo", algo)
            o = run_attention(q, k, v, chains, algo)
            assert not np.isnan(o).any()
            errs[(algo, chains)] = R.rel_error(o, ref)
    ratios = {a: errs[(a, 1)] / errs[(a, 2)] for a in algos if (a, 1) in errs and (a, 2) in errs}
    print(f"attention 2048 x {nk}: errors (algo, chains) {errs}; 1-chain / 2-chain ratio per algo {ratios}")
    return errs


def test_attention_full_size():
    """The 2048 x 32768 x 128 workload: all 2048 query rows against the oracle,
    both algorithms, one and two chains, each within 5e-6."""
    errs = _all_rows(32768)
    for key, e in errs.items():
        assert e <= 5e-6, key


@pytest.mark.parametrize("nk", [8192, 131072])
def test_attention_page_contexts(nk):
    """The other two contexts of Strata PR #800's "Numbers" table (2,048 queries
    at 8,192 and 131,072 keys): one and two chains through both algorithms,
    every row against the oracle.  The page reports 5.88e-6 / 5.35e-6 for one
    chain and 3.02e-6 / 2.75e-6 for two on its hardware; here both must stay
    within 5e-6."""
    errs = _all_rows(nk)
    for key, e in errs.items():
        assert e <= 5e-6, key


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
    """2048 x 32768, all rows: against the reference on the ORIGINAL K and V,
    rounding K and V once (algo 1) leaves an error floor; splitting them (algo
    2) removes it."""
    q, k, v = inputs.attention()
    ref = R.attention_ref(q, k, v, round_kv=False)
    errs = {}
    for algo in (mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV):
        for chains in (1, 2):
            say("attention vs fp32 K/V reference", algo, chains)
            o = run_attention(q, k, v, chains, algo)
            assert not np.isnan(o).any()
            errs[(algo, chains)] = R.rel_error(o, ref)
    print("errors against the fp32-K/V reference (algo, chains):", errs)
    assert errs[(mfl.ATTN_FUSED_SPLIT_KV, 2)] <= 5e-6
    assert errs[(mfl.ATTN_FUSED_SPLIT_KV, 1)] <= 5e-6
    assert errs[(mfl.ATTN_FUSED, 2)] >= 10 * errs[(mfl.ATTN_FUSED_SPLIT_KV, 2)]


# The largest key count the fused kernels take (nk * 128 * 2 bytes of K16 within
# a 32-bit buffer extent): 2^24 - 128 keys, one block of 128 queries.  With
# K = 0 every score is 0, P~ = 1 and O is the mean of the V rows; V's rows are
# 1 + j/8 (j = bits 16-18 of the key index), exact in fp16, so every partial
# sum of the kernels is an integer below 2^24 and the result is the exact mean
# up to the last fp32 roundings.  A key counted twice, skipped, or read from
# the wrong place past 2^23 keys changes the mean.
@pytest.mark.parametrize("algo", [mfl.ATTN_MATERIALISED, mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV])
def test_attention_maximum_keys(algo):
    nq, nk, d = 128, (1 << 24) - 128, 128
    say("attention maximum keys", algo, nk)
    kidx = torch.arange(nk, device=device())
    vcol = 1.0 + ((kidx >> 16) & 7).to(torch.float32) / 8.0
    v = vcol[:, None].expand(nk, d).contiguous()
    del kidx, vcol
    k = torch.zeros((nk, d), device=device())
    q = torch.from_numpy(np.random.default_rng(5).standard_normal((nq, d)).astype(np.float32)).to(device())
    wsb = mfl.attention_workspace_bytes(nq, nk, d, algo)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device())
    o = torch.full((nq, d), np.nan, device=device())
    mfl.attention_split_fp32(nq, nk, d, q, k, v, 2, algo, o, ws, wsb, stream())
    out = host(o)
    del ws, k, v
    torch.cuda.empty_cache()
    full, rest = divmod(nk, 1 << 16)
    total = sum((8 + (b & 7)) * (1 << 16) for b in range(full)) + (8 + (full & 7)) * rest   # in eighths
    want = total / 8.0 / nk
    assert not np.isnan(out).any()
    assert np.max(np.abs(out - want)) <= 1e-6 * want
