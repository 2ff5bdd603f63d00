"""gemm_tile_mma against the oracle: fp64 product of the quantised inputs,
normwise relative error <= 1e-5; bit-exact on integer-valued inputs; all four
operand orders; every tile configuration of the fast path (64, 128, 192 and
256 wide); ragged edges; NaN padding never read; the 4096^3 bf16 case in the
launch configuration the benchmark times (every element of C)."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from mma_fragment_layouts_amd import inputs
from oracle import reference as R

from _gpu import DT, dev32, device, host, q16, say, stream

pytestmark = pytest.mark.gpu
TOL = 1e-5
SENTINEL = 12345.0


def storage(x_logical, order, ld, pad_value=np.nan):
    """Storage array of a logical matrix in the given order and leading dim."""
    if order == mfl.ROW_MAJOR:
        rows, cols = x_logical.shape
        s = np.full((rows, ld), pad_value, np.float32)
        s[:, :cols] = x_logical
    else:
        cols, rows = x_logical.shape[1], x_logical.shape[0]
        s = np.full((cols, ld), pad_value, np.float32)
        s[:, :rows] = x_logical.T
    return s


def run_gemm(fmt, a, b, order_a=mfl.ROW_MAJOR, order_b=mfl.COL_MAJOR, pad=8, shape=None, accumulate=0, c0=None):
    """a: logical M x K, b: logical K x N (fp32 numpy).  Returns C (numpy)."""
    m, k = a.shape
    n = b.shape[1]
    lda = (k if order_a == mfl.ROW_MAJOR else m) + pad
    ldb = (n if order_b == mfl.ROW_MAJOR else k) + pad
    lda += (-lda) % 8
    ldb += (-ldb) % 8
    sa = storage(a, order_a, lda)
    sb = storage(b, order_b, ldb)
    da, db = q16(sa, fmt), q16(sb, fmt)
    c = dev32(c0) if c0 is not None else torch.full((m, n), np.nan, device=device())
    if shape is None:
        mfl.gemm_tile_mma(DT[fmt], m, n, k, da, lda, order_a, db, ldb, order_b, c, n, accumulate, stream())
    else:
        mfl.gemm_tile_mma_shape(shape, DT[fmt], m, n, k, da, lda, order_a, db, ldb, order_b, c, n, accumulate,
                                stream())
    return host(c)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm_small_config(fmt):
    """M = N = K = 256, uniform[-1, 1], A row-major, B column-major."""
    a, bt = inputs.gemm_small()
    assert not np.array_equal(a, bt)
    say("gemm 256^3", fmt)
    c = run_gemm(fmt, a, bt.T)
    assert R.rel_error(c, R.gemm_ref(a, bt, fmt)) <= TOL


@pytest.mark.parametrize("oa", [mfl.ROW_MAJOR, mfl.COL_MAJOR])
@pytest.mark.parametrize("ob", [mfl.ROW_MAJOR, mfl.COL_MAJOR])
def test_all_operand_orders(oa, ob):
    a, bt = inputs.gemm_small()
    say("gemm orders", oa, ob)
    c = run_gemm("f16", a, bt.T, oa, ob)
    assert R.rel_error(c, R.gemm_ref(a, bt, "f16")) <= TOL


def test_wrong_declared_order_gives_a_different_product():
    """Declaring the wrong layout computes another product without any
    out-of-bounds access (explainer, paragraph on leading dimensions)."""
    a, bt = inputs.gemm_small()
    c = run_gemm("f16", a, bt.T)
    sa = storage(a, mfl.ROW_MAJOR, 256)
    sb = storage(bt.T, mfl.COL_MAJOR, 256)
    cc = torch.empty((256, 256), device=device())
    mfl.gemm_tile_mma(mfl.F16, 256, 256, 256, q16(sa, "f16"), 256, mfl.COL_MAJOR, q16(sb, "f16"), 256,
                      mfl.COL_MAJOR, cc, 256, 0, stream())
    assert R.rel_error(host(cc), c) > 0.5


@pytest.mark.parametrize("mnk", [(200, 136, 100), (129, 257, 72), (1, 1, 1), (17, 300, 8), (384, 384, 1000),
                                 (256, 512, 130)])
@pytest.mark.parametrize("orders", [(0, 1), (1, 0), (0, 0), (1, 1)])
def test_ragged_sizes(mnk, orders):
    m, n, k = mnk
    rng = np.random.default_rng(m * 7 + n * 3 + k)
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    b = rng.uniform(-1, 1, (k, n)).astype(np.float32)
    say("gemm ragged", mnk, orders)
    c = run_gemm("bf16", a, b, *orders)
    assert not np.isnan(c).any()
    assert R.rel_error(c, R.gemm_ref(a, b.T, "bf16")) <= TOL


def test_integer_inputs_are_bit_exact():
    rng = np.random.default_rng(9)
    m, n, k = 512, 512, 512
    a = rng.integers(-16, 17, (m, k)).astype(np.float32)
    b = rng.integers(-16, 17, (k, n)).astype(np.float32)
    exact = a.astype(np.int64) @ b.astype(np.int64)
    for shape in (0, 1):
        say("gemm integer exact", shape)
        c = run_gemm("bf16", a, b, shape=shape)
        assert np.array_equal(c, exact.astype(np.float32))


def test_accumulate_and_k_zero():
    rng = np.random.default_rng(10)
    a = rng.uniform(-1, 1, (256, 192)).astype(np.float32)
    b = rng.uniform(-1, 1, (192, 320)).astype(np.float32)
    c0 = rng.uniform(-1, 1, (256, 320)).astype(np.float32)
    say("gemm accumulate")
    c = run_gemm("f16", a, b, accumulate=1, c0=c0)
    assert R.rel_error(c, c0 + R.gemm_ref(a, b.T, "f16")) <= TOL
    say("gemm K = 0")
    z = torch.full((64, 64), 3.0, device=device())
    mfl.gemm_tile_mma(mfl.F16, 64, 64, 0, 0, 8, 0, 0, 8, 1, z, 64, 0, stream())
    assert np.all(host(z) == 0)
    mfl.gemm_tile_mma(mfl.F16, 64, 64, 0, 0, 8, 0, 0, 8, 1, z, 64, 1, stream())
    assert np.all(host(z) == 0)


@pytest.mark.parametrize("shape", [0, 1])
def test_fast_path_padded_nan(shape):
    """Fast path (256-multiples, K-contiguous) with NaN in the padding of both
    operands: a single read of the padding would poison the output."""
    a, bt = inputs.gemm_dense(512, 768, 1024, pad=64)
    say("fast path nan pad", shape)
    c = torch.full((512, 768), np.nan, device=device())
    mfl.gemm_tile_mma_shape(shape, mfl.BF16, 512, 768, 1024, q16(a, "bf16"), 1088, mfl.ROW_MAJOR, q16(bt, "bf16"),
                            1088, mfl.COL_MAJOR, c, 768, 0, stream())
    ch = host(c)
    assert not np.isnan(ch).any()
    assert R.rel_error(ch, R.gemm_ref(a[:, :1024], bt[:, :1024], "bf16")) <= TOL


_DENSE_REF = {}


def dense_4096_ref(a, bt, fmt):
    """The oracle's fp64 product of the quantised 4096^3 operands (computed once
    per 16-bit format and kept for the other instruction shape)."""
    if fmt not in _DENSE_REF:
        _DENSE_REF[fmt] = R.gemm_ref(a[:, :4096], bt[:, :4096], fmt)
    return _DENSE_REF[fmt]


@pytest.mark.parametrize("shape,fmt", [(0, "bf16"), (1, "bf16"), (0, "f16"), (1, "f16")])
def test_dense_4096_full(shape, fmt):
    """The 4096^3 GEMM exactly as the benchmark launches it (A row-major, B
    column-major, ld 4160 with NaN padding, C fp32 ldc 4096), in bf16 and, as
    the benchmark's variant leg runs it, fp16: no NaN anywhere; every element
    of C against the oracle, normwise within 1e-5; and 4096 sampled entries
    elementwise against single dot products of the oracle."""
    a, bt = inputs.gemm_dense()
    say("dense 4096^3", shape, fmt)
    c = torch.full((4096, 4096), np.nan, device=device())
    mfl.gemm_tile_mma_shape(shape, DT[fmt], 4096, 4096, 4096, q16(a, fmt), 4160, mfl.ROW_MAJOR,
                            q16(bt, fmt), 4160, mfl.COL_MAJOR, c, 4096, 0, stream())
    ch = host(c)
    assert not np.isnan(ch).any()
    err = R.rel_error(ch, dense_4096_ref(a, bt, fmt))
    print(f"dense 4096^3 shape={shape} {fmt}: normwise error over all of C {err:.3e}")
    assert err <= TOL
    rng = np.random.default_rng(11)
    r = rng.integers(0, 4096, 4096)
    cc = rng.integers(0, 4096, 4096)
    ref = R.gemm_ref_entries(a[:, :4096], bt[:, :4096], fmt, r, cc)
    # elementwise: fp32 accumulation of 4096 products, bound ~ K * u32 * sum|a||b|
    scale = np.abs(ref).max()
    assert np.max(np.abs(ch[r, cc] - ref)) <= 4096 * 2.0 ** -24 * 64 * max(scale, 1.0)


# The fast path picks its tile by problem size: 64 x 64 (2 waves) for small
# problems, 128 x 128 (4 waves) in between, 256 x 256 (16 waves) from 128 such
# tiles up.  Each size below lands on one of them (comment), with both MFMA
# instructions and both 16-bit types; accumulate on for one of each.
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("mnk,accumulate", [((256, 256, 256), 0),     # 32 x 32 (64 x 64 with 32x32x16)
                                             ((192, 320, 128), 1),     # 32 x 32, ragged for 64 and 128
                                             ((512, 768, 256), 0),     # 32 x 32, 384 workgroups
                                             ((1024, 1024, 512), 0),   # 64 x 64, 256 workgroups
                                             ((2048, 2048, 256), 1),   # 128 x 128, 256 workgroups
                                             ((2048, 4096, 128), 0),   # 256 x 256, 128 workgroups
                                             ((3072, 3072, 3072), 0),  # 192 x 192 (16x16x32), 256 workgroups
                                             ((3072, 3072, 512), 1)])
def test_fast_path_tile_sizes(mnk, accumulate, shape, fmt):
    m, n, k = mnk
    rng = np.random.default_rng(m + n + k + shape)
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    bt = rng.uniform(-1, 1, (n, k)).astype(np.float32)
    c0 = rng.standard_normal((m, n)).astype(np.float32) if accumulate else None
    say("gemm fast tiles", m, n, k, shape, fmt, accumulate)
    c = run_gemm(fmt, a, bt.T, shape=shape, accumulate=accumulate, c0=c0)
    ref = R.gemm_ref(a, bt, fmt) + (c0.astype(np.float64) if accumulate else 0.0)
    assert not np.isnan(c).any()
    assert R.rel_error(c, ref) <= TOL


# K-strided operands (A column-major, B row-major) take the fast path through
# k-major LDS slabs read with the gfx950 transpose read.  Every lane still holds
# the K positions of the operand numeral and the MFMA sequence is the same, so
# each order gives the same bits as the K-contiguous launch on the same values.
ORDERS = [(mfl.ROW_MAJOR, mfl.COL_MAJOR), (mfl.ROW_MAJOR, mfl.ROW_MAJOR), (mfl.COL_MAJOR, mfl.COL_MAJOR),
          (mfl.COL_MAJOR, mfl.ROW_MAJOR)]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("mnk,accumulate", [((4096, 4096, 128), 0),   # 256 x 256 tiles
                                            ((2048, 1024, 192), 0),   # 128 x 128 tiles
                                            ((3072, 3072, 256), 1),   # 192 x 192 (K-contiguous, 16x16x32), 256 x 256
                                            ((256, 384, 320), 1),     # 128 x 128 (k-major), 32 x 32 (K-contiguous)
                                            ((128, 128, 64), 0)])     # one tile, one K step
def test_fast_path_all_orders_bit_identical(mnk, accumulate, shape, fmt):
    m, n, k = mnk
    rng = np.random.default_rng(3 * m + n + k + shape)
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    b = rng.uniform(-1, 1, (k, n)).astype(np.float32)
    c0 = rng.standard_normal((m, n)).astype(np.float32) if accumulate else None
    ref = R.gemm_ref(a, np.ascontiguousarray(b.T), fmt) + (c0.astype(np.float64) if accumulate else 0.0)
    first = None
    for oa, ob in ORDERS:
        say("gemm fast orders", m, n, k, shape, fmt, oa, ob)
        c = run_gemm(fmt, a, b, oa, ob, shape=shape, accumulate=accumulate, c0=c0)
        assert not np.isnan(c).any()
        assert R.rel_error(c, ref) <= TOL
        if first is None:
            first = c
        else:
            assert np.array_equal(c.view(np.uint32), first.view(np.uint32)), (oa, ob)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("orders", ORDERS[1:])
def test_dense_4096_bf16_other_orders(orders, shape):
    """The benchmark's 4096^3 bf16 GEMM with K-strided operands (ld 4160, NaN
    padding): bit-identical to the K-contiguous launch on the same values."""
    a, bt = inputs.gemm_dense()
    n = 4096

    def padded(x):
        s = np.full((n, 4160), np.nan, np.float32)
        s[:, :n] = x
        return s

    oa, ob = orders
    sa = a if oa == mfl.ROW_MAJOR else padded(a[:, :n].T)
    sb = bt if ob == mfl.COL_MAJOR else padded(bt[:, :n].T)
    say("dense 4096^3 orders", oa, ob, shape)
    ref = torch.empty((n, n), device=device())
    mfl.gemm_tile_mma_shape(shape, mfl.BF16, n, n, n, q16(a, "bf16"), 4160, mfl.ROW_MAJOR, q16(bt, "bf16"), 4160,
                            mfl.COL_MAJOR, ref, n, 0, stream())
    c = torch.full((n, n), np.nan, device=device())
    mfl.gemm_tile_mma_shape(shape, mfl.BF16, n, n, n, q16(sa, "bf16"), 4160, oa, q16(sb, "bf16"), 4160, ob, c, n, 0,
                            stream())
    assert torch.equal(c.view(torch.int32), ref.view(torch.int32))


# Sizes that are not tile multiples (K a multiple of 8) run the fast kernel's
# EDGE variant: loads past M / N return zeros (or neighbouring storage) through
# the buffer extents, K positions past K are zeroed in the registers, and only
# elements inside C are stored.  C here has
# ldc = N + 5 with a sentinel in its padding, which must survive; every order
# must still give the same bits.
@pytest.mark.parametrize("fmt", ["bf16", "f16"])
@pytest.mark.parametrize("mnk,accumulate", [((200, 136, 128), 0),      # 32 x 32 tiles (K-contiguous), 128 (k-major)
                                            ((1000, 520, 192), 1),
                                            ((8, 264, 64), 0),         # fewer rows than one tile
                                            ((4000, 4000, 256), 0),    # 256 x 256 tiles, ragged last row / column
                                            ((2056, 1160, 128), 1),
                                            ((1000, 520, 200), 0),     # K not a multiple of 64: masked last slab
                                            ((264, 136, 8), 1),        # a single partial K slab
                                            ((4000, 4096, 4040), 0),   # 256 x 256 tiles, every edge ragged
                                            ((2904, 3000, 1000), 1),   # 192 x 192 (K-contiguous), 256 x 256
                                            ((3072, 2824, 200), 0)])   # 192 x 192 with ragged N and K
def test_fast_path_ragged_all_orders(mnk, accumulate, fmt):
    m, n, k = mnk
    rng = np.random.default_rng(m + 7 * n + k)
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    b = rng.uniform(-1, 1, (k, n)).astype(np.float32)
    ldc = n + 5
    c0 = rng.standard_normal((m, n)).astype(np.float32)
    ref = R.gemm_ref(a, np.ascontiguousarray(b.T), fmt) + (c0.astype(np.float64) if accumulate else 0.0)
    first = None
    for oa, ob in ORDERS:
        say("gemm fast ragged", m, n, k, fmt, accumulate, oa, ob)
        sa = storage(a, oa, (k if oa == mfl.ROW_MAJOR else m) + 8)
        sb = storage(b, ob, (n if ob == mfl.ROW_MAJOR else k) + 8)
        cs = np.full((m, ldc), 12345.0, np.float32)
        cs[:, :n] = c0 if accumulate else np.nan
        c = dev32(cs)
        mfl.gemm_tile_mma(DT[fmt], m, n, k, q16(sa, fmt), sa.shape[1], oa, q16(sb, fmt), sb.shape[1], ob, c, ldc,
                          accumulate, stream())
        ch = host(c)
        assert np.all(ch[:, n:] == 12345.0), "padding of C was written"
        out = ch[:, :n]
        assert not np.isnan(out).any()
        assert R.rel_error(out, ref) <= TOL
        if first is None:
            first = out.copy()
        else:
            assert np.array_equal(out.view(np.uint32), first.view(np.uint32)), (oa, ob)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("accumulate", [0, 1])
@pytest.mark.parametrize("m,n,k", [(6144, 6144, 6144), (6000, 6100, 2000)])
def test_wave_quantisation_split(m, n, k, shape, accumulate):
    """Sizes with two full rounds of 256 x 256 tiles on 256 CUs and a partial
    one run as two launches: rows 0-5119 with 256-tiles, the rest with
    128-tiles (6144^3: 576 tiles; 6000 x 6100 x 2000: 24 x 24 tiles, ragged M,
    N and a K tail, so both launches run their EDGE variants).  Row blocks of
    both regions and the block across the boundary, recomputed by standalone
    calls on those rows alone, must match bit for bit (the tile size does not
    change an element's MFMA sequence); sampled rows of both regions against
    the oracle; the padding of C untouched."""
    ldc = n + 4
    a, bt = inputs.gemm_dense(m, n, k)
    ld = a.shape[1]
    say("quantisation split", m, n, k, shape, accumulate)
    da, db = q16(a, "bf16"), q16(bt, "bf16")
    rng = np.random.default_rng(21)
    c0 = np.full((m, ldc), SENTINEL, np.float32)
    c0[:, :n] = rng.standard_normal((m, n)).astype(np.float32) if accumulate else np.nan
    c = dev32(c0)
    mfl.gemm_tile_mma_shape(shape, mfl.BF16, m, n, k, da, ld, mfl.ROW_MAJOR, db, ld, mfl.COL_MAJOR, c, ldc,
                            accumulate, stream())
    ch = host(c)
    assert (ch[:, n:] == SENTINEL).all(), "C padding written"
    assert not np.isnan(ch[:, :n]).any()
    for r0, rows in ((0, 256), (4992, 256), (m - 200, 200)):    # main region, across the boundary, rest
        part = dev32(c0[r0:r0 + rows])
        mfl.gemm_tile_mma_shape(shape, mfl.BF16, rows, n, k, da[r0:], ld, mfl.ROW_MAJOR, db, ld, mfl.COL_MAJOR,
                                part, ldc, accumulate, stream())
        assert np.array_equal(host(part)[:, :n].view(np.uint32), ch[r0:r0 + rows, :n].view(np.uint32)), r0
    sample = np.concatenate([rng.choice(5120, 12, replace=False), 5120 + rng.choice(m - 5120, 12, replace=False)])
    ref = R.gemm_ref(a[sample, :k], bt[:, :k], "bf16") + (c0[sample, :n].astype(np.float64) if accumulate else 0.0)
    assert R.rel_error(ch[sample, :n], ref) <= TOL


@pytest.mark.parametrize("m,n,k", [(6144, 6144, 2048), (6000, 6104, 2000)])
@pytest.mark.parametrize("oa,ob", [(mfl.COL_MAJOR, mfl.COL_MAJOR), (mfl.ROW_MAJOR, mfl.ROW_MAJOR),
                                   (mfl.COL_MAJOR, mfl.ROW_MAJOR)])
def test_wave_quantisation_split_k_major(oa, ob, m, n, k):
    """The row split with k-major operands (column-major A: the second launch
    starts M1 elements in; row-major B): 6144 x 6144 x 2048, and 6000 x 6104 x
    2000 where M, N and K are all ragged so both launches run their EDGE
    variants on the offset column-major A.  Bit-identical to the K-contiguous
    order (same MFMA sequence per element) and, per row block (the first rows,
    the block across the boundary at row 5120, the last rows), to standalone
    calls on those rows; sampled rows against the oracle."""
    a, bt = inputs.gemm_dense(m, n, k)
    a, bt = a[:, :k], bt[:, :k]
    say("quantisation split k-major", oa, ob, m, n, k)
    sa = a if oa == mfl.ROW_MAJOR else np.ascontiguousarray(a.T)      # storage: rows x inner
    sb = bt if ob == mfl.COL_MAJOR else np.ascontiguousarray(bt.T)
    da, db = q16(sa, "bf16"), q16(sb, "bf16")
    lda, ldb = sa.shape[1], sb.shape[1]
    c_ref = torch.full((m, n), np.nan, device=device())
    mfl.gemm_tile_mma(mfl.BF16, m, n, k, q16(a, "bf16"), k, mfl.ROW_MAJOR, q16(bt, "bf16"), k, mfl.COL_MAJOR, c_ref,
                      n, 0, stream())
    c = torch.full((m, n), np.nan, device=device())
    mfl.gemm_tile_mma(mfl.BF16, m, n, k, da, lda, oa, db, ldb, ob, c, n, 0, stream())
    assert not torch.isnan(c).any()
    assert torch.equal(c, c_ref)
    for r0 in (0, 4992, m - 256):
        part = torch.full((256, n), np.nan, device=device())
        sub_a = da[r0:] if oa == mfl.ROW_MAJOR else da[:, r0:]         # rows r0.. of A
        mfl.gemm_tile_mma(mfl.BF16, 256, n, k, sub_a, lda, oa, db, ldb, ob, part, n, 0, stream())
        assert torch.equal(part, c[r0:r0 + 256]), r0
    rows = np.random.default_rng(22).choice(m, 16, replace=False)
    assert R.rel_error(host(c)[rows], R.gemm_ref(a[rows], bt, "bf16")) <= TOL


# Leading dimensions at the fast path's 32-bit buffer-offset limit.  The fast
# path addresses an operand through a 32-bit buffer extent (a K-contiguous
# operand: one panel of at most 256 rows; a k-major one: all K rows) and C
# through 256 rows of ldc; just below those limits it still runs, at or past
# them the dispatcher takes the generic path, whose addresses are 64-bit.  The
# storage here is 4-4.3 GiB per operand; only the M x K (K x N) block is set.
@pytest.mark.parametrize("side", ["below", "past"])
@pytest.mark.parametrize("oa,ob", [(mfl.ROW_MAJOR, mfl.COL_MAJOR), (mfl.COL_MAJOR, mfl.ROW_MAJOR)])
def test_leading_dimensions_at_the_32_bit_limit(side, oa, ob):
    m = n = k = 256
    ld = (1 << 23) - 64 if side == "below" else (1 << 23) + 64   # 256 * ld * 2 bytes vs 2^32
    ldc = (1 << 22) - 64 if side == "below" else (1 << 22) + 64  # 256 * ldc * 4 bytes vs 2^32
    rng = np.random.default_rng(41 + (side == "past"))
    a = rng.uniform(-1, 1, (m, k)).astype(np.float32)
    b = rng.uniform(-1, 1, (k, n)).astype(np.float32)
    ref = R.gemm_ref(a, np.ascontiguousarray(b.T), "bf16")

    def big(x_logical, order):
        """Device storage rows x ld (bf16, zeros) holding the logical matrix in `order`."""
        block = x_logical if order == mfl.ROW_MAJOR else np.ascontiguousarray(x_logical.T)
        s = torch.zeros((block.shape[0], ld), dtype=torch.int16, device=device())
        s[:, : block.shape[1]] = q16(block, "bf16")
        return s

    say("gemm ld at 32-bit limit", side, oa, ob, ld, ldc)
    sa, sb = big(a, oa), big(b, ob)
    c = torch.full((m, ldc), SENTINEL, device=device())
    c[:, :n] = np.nan
    mfl.gemm_tile_mma(mfl.BF16, m, n, k, sa, ld, oa, sb, ld, ob, c, ldc, 0, stream())
    out = host(c[:, :n])
    assert not np.isnan(out).any()
    assert R.rel_error(out, ref) <= TOL
    assert bool((c[:, n:] == SENTINEL).all()), "padding of C was written"
    # the same values through compact storage give the same bits
    small = run_gemm("bf16", a, b, oa, ob)
    assert np.array_equal(out.view(np.uint32), small.view(np.uint32))
    del sa, sb, c
    torch.cuda.empty_cache()
