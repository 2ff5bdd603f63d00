"""HIP graph capture of the library's device entry points.

Every device entry point only launches kernels on the caller's stream: no
allocation, copy, fill or synchronisation.  So a caller can capture a call in a
graph (a serving loop, a launch-bound sequence of small products) and replay
it.  Each test captures a call on a side stream, replays the graph several
times with the program's own eager work and synchronisations in between, and
checks every replay bit for bit against the same call made eagerly."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from mma_fragment_layouts_amd import inputs

from _gpu import dev32, device, q16, say, stream

pytestmark = pytest.mark.gpu
REPLAYS = 4


def capture(call):
    """Capture call(stream) into a graph on a side stream of default priority."""
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=side):
        call(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return g


def eager_noise(shape):
    """Unrelated eager work between replays: a fill and a small product."""
    x = torch.full(shape, 3.0, device=device())
    y = x @ x.T[:, : shape[0]].contiguous()
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("mnk,orders", [((2048, 1536, 1024), (mfl.ROW_MAJOR, mfl.COL_MAJOR)),
                                        ((1000, 520, 200), (mfl.COL_MAJOR, mfl.ROW_MAJOR)),
                                        ((256, 256, 256), (mfl.ROW_MAJOR, mfl.COL_MAJOR)),
                                        # 24 x 24 tiles of 256: the row split, two launches per call
                                        ((6144, 6144, 1024), (mfl.ROW_MAJOR, mfl.COL_MAJOR))])
def test_graph_gemm_tile_mma(mnk, orders):
    m, n, k = mnk
    oa, ob = orders
    rng = np.random.default_rng(m + n + k)
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    bt = rng.uniform(-1, 1, (n, k)).astype(np.float32)
    sa = a if oa == mfl.ROW_MAJOR else np.ascontiguousarray(a.T)
    sb = bt if ob == mfl.COL_MAJOR else np.ascontiguousarray(bt.T)
    da, db = q16(sa, "bf16"), q16(sb, "bf16")
    lda, ldb = sa.shape[1], sb.shape[1]
    say("graph gemm", mnk, orders)

    def call(c, accumulate, st):
        mfl.gemm_tile_mma(mfl.BF16, m, n, k, da, lda, oa, db, ldb, ob, c, n, accumulate, st)

    # overwrite: every replay equals the eager result
    c_eager = torch.full((m, n), np.nan, device=device())
    call(c_eager, 0, stream())
    c_graph = torch.empty((m, n), device=device())
    g = capture(lambda st: call(c_graph, 0, st))
    for r in range(REPLAYS):
        c_graph.fill_(np.nan)
        eager_noise((64, 64))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c_graph, c_eager), f"replay {r}"

    # accumulate: replay r equals r + 1 eager accumulating calls from the same start
    c0 = dev32(rng.standard_normal((m, n)).astype(np.float32))
    c_eager, c_graph = c0.clone(), c0.clone()
    g = capture(lambda st: call(c_graph, 1, st))
    c_graph.copy_(c0)
    for r in range(REPLAYS):
        call(c_eager, 1, stream())
        eager_noise((32, 32))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c_graph, c_eager), f"accumulating replay {r}"


@pytest.mark.parametrize("mnk", [(512, 384, 640), (1000, 520, 200)])
def test_graph_split_planes(mnk):
    """gemm_split_fp32_ws on the planes path: two split kernels and the GEMM."""
    m, n, k = mnk
    a, bt = inputs.gemm_split(m, n, k)
    lda = ldb = k + (-k) % 8
    pa = np.full((m, lda), np.nan, np.float32)
    pa[:, :k] = a
    pb = np.full((n, ldb), np.nan, np.float32)
    pb[:, :k] = bt
    da, db = dev32(pa), dev32(pb)
    wsb = mfl.gemm_split_fp32_workspace_bytes(m, n, k, lda, mfl.ROW_MAJOR, mfl.SPLIT, ldb, mfl.COL_MAJOR, mfl.SPLIT, n)
    assert wsb > 0
    ws = torch.empty(wsb, dtype=torch.uint8, device=device())
    say("graph split planes", mnk)

    def call(c, st):
        mfl.gemm_split_fp32_ws(mfl.BF16, m, n, k, da, lda, mfl.ROW_MAJOR, mfl.SPLIT, db, ldb, mfl.COL_MAJOR,
                               mfl.SPLIT, 2, 0, c, n, 0, ws, wsb, st)

    c_eager = torch.full((m, n), np.nan, device=device())
    call(c_eager, stream())
    torch.cuda.synchronize()
    c_graph = torch.empty((m, n), device=device())
    g = capture(lambda st: call(c_graph, st))
    for r in range(REPLAYS):
        c_graph.fill_(np.nan)
        ws.zero_()  # the replay must rebuild its planes
        eager_noise((64, 64))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c_graph, c_eager), f"replay {r}"


@pytest.mark.parametrize("algo", [mfl.ATTN_MATERIALISED, mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV])
def test_graph_attention(algo):
    """attention_split_fp32: preparation, the per-slice kernel and the combine."""
    nq, nk, d = 256, 4096, 128
    q, k, v = (dev32(x) for x in inputs.attention(nq, nk))
    wsb = mfl.attention_workspace_bytes(nq, nk, d, algo)
    ws = torch.empty(wsb, dtype=torch.uint8, device=device())
    say("graph attention", algo)

    def call(o, st):
        mfl.attention_split_fp32(nq, nk, d, q, k, v, 2, algo, o, ws, wsb, st)

    o_eager = torch.full((nq, d), np.nan, device=device())
    call(o_eager, stream())
    torch.cuda.synchronize()
    o_graph = torch.empty((nq, d), device=device())
    g = capture(lambda st: call(o_graph, st))
    for r in range(REPLAYS):
        o_graph.fill_(np.nan)
        ws.zero_()
        eager_noise((64, 64))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {r}"


@pytest.mark.parametrize("algo", [mfl.ATTN_MATERIALISED, mfl.ATTN_FUSED, mfl.ATTN_FUSED_SPLIT_KV])
def test_graph_attention_static(algo):
    """attention_split_fp32_static, the entry point for callers that cannot
    allocate: its workspace is the library's static device array, so the
    captured graph holds only kernel launches on that array."""
    nq, nk, d = 256, 4096, 128
    q, k, v = (dev32(x) for x in inputs.attention(nq, nk))
    say("graph attention static", algo)

    def call(o, st):
        mfl.attention_split_fp32_static(nq, nk, d, q, k, v, 2, algo, o, st)

    o_eager = torch.full((nq, d), np.nan, device=device())
    call(o_eager, stream())
    torch.cuda.synchronize()
    o_graph = torch.empty((nq, d), device=device())
    g = capture(lambda st: call(o_graph, st))
    for r in range(REPLAYS):
        o_graph.fill_(np.nan)
        eager_noise((64, 64))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_graph, o_eager), f"replay {r}"
