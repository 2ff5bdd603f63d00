"""Device checks of the accumulator layouts against the hardware (cuda-oxide PR
#474, "Verified against hardware"): one raw MFMA per instruction and operand
type, operands gathered on the host, registers compared through the oracle's
enumerated layout.  Expected values are exact integers computed on the host."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from oracle import layouts as OL

import mfma_sum_model as MODEL
from _gpu import DT, device, host, q16, say, stream

pytestmark = pytest.mark.gpu

GEOM = {0: (OL.MFMA_16X16X32, 16, 32), 1: (OL.MFMA_32X32X16, 32, 16)}  # map, MN, K


def gather(a, b, mn):
    """Operand fragments: lane l holds A[l % mn][8*(l // mn) + i] and
    B[8*(l // mn) + i][l % mn], i = 0..7 (the CDNA4 operand layout of these
    instructions)."""
    af = np.zeros((64, 8), np.float32)
    bf = np.zeros((64, 8), np.float32)
    for l in range(64):
        for i in range(8):
            af[l, i] = a[l % mn, 8 * (l // mn) + i]
            bf[l, i] = b[8 * (l // mn) + i, l % mn]
    return af, bf


def run_probe(shape, fmt, a, b, c_in=None):
    fm, mn, k = GEOM[shape]
    af, bf = gather(a, b, mn)
    dev = device()
    at = torch.from_numpy(af.reshape(-1)).to(dev)
    bt = torch.from_numpy(bf.reshape(-1)).to(dev)
    a16 = torch.empty(64 * 8, dtype=torch.int16, device=dev)
    b16 = torch.empty(64 * 8, dtype=torch.int16, device=dev)
    mfl.quantize_fp32(DT[fmt], at, a16, 64 * 8, stream())
    mfl.quantize_fp32(DT[fmt], bt, b16, 64 * 8, stream())
    acc = torch.full((64 * fm.per_lane,), float("nan"), device=dev)
    cin = None
    if c_in is not None:   # c_in: logical mn x mn matrix, handed over lane-major through the oracle layout
        lm = np.zeros((64, fm.per_lane), np.float32)
        for l in range(64):
            for j in range(fm.per_lane):
                lm[l, j] = c_in[fm.coords(l, j)]
        cin = torch.from_numpy(lm.reshape(-1)).to(dev)
    mfl.mfma_probe(shape, DT[fmt], a16, b16, cin, acc, stream())
    return host(acc).reshape(64, fm.per_lane)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [0, 1])
def test_identity_decode(shape, fmt):
    """B = identity on a window of columns, A encodes its row (or column) index:
    each register then names the output position it holds."""
    fm, mn, k = GEOM[shape]
    kw = min(k, mn)
    mism = 0
    for h in range(mn // kw):
        for enc in ("row", "col"):
            say("identity decode", shape, fmt, h, enc)
            a = np.zeros((mn, k), np.float32)
            b = np.zeros((k, mn), np.float32)
            for r in range(mn):
                for kk in range(kw):
                    a[r, kk] = r + 1 if enc == "row" else kk + 1
            for kk in range(kw):
                b[kk, h * kw + kk] = 1.0
            acc = run_probe(shape, fmt, a, b)
            for l in range(64):
                for j in range(fm.per_lane):
                    r, c = fm.coords(l, j)
                    inwin = h * kw <= c < (h + 1) * kw
                    want = (r + 1 if enc == "row" else c - h * kw + 1) if inwin else 0.0
                    mism += acc[l, j] != want
    assert mism == 0, f"{mism} mismatched registers"


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [0, 1])
def test_asymmetric_integer_matmul(shape, fmt):
    """Distinct integers +-1..+-256 in A and a different arrangement in B: every
    partial sum is an exact fp32 integer, so the product is bit-exact under any
    accumulation order; a transposed or half-swapped layout cannot match."""
    fm, mn, k = GEOM[shape]
    rng = np.random.default_rng(100 + shape)
    pool = np.array([v for v in range(-256, 257) if v != 0], np.float32)
    a = rng.permutation(pool)[: mn * k].reshape(mn, k)
    b = rng.permutation(pool)[: k * mn].reshape(k, mn)
    assert not np.array_equal(a, b.T)
    exact = (a.astype(np.int64) @ b.astype(np.int64)).astype(np.float64)
    say("asymmetric matmul", shape, fmt)
    acc = run_probe(shape, fmt, a, b)
    mism, worst = 0, 0.0
    for l in range(64):
        for j in range(fm.per_lane):
            r, c = fm.coords(l, j)
            d = abs(float(acc[l, j]) - exact[r, c])
            mism += d != 0
            worst = max(worst, d)
    assert (mism, worst) == (0, 0.0), f"{mism}/{64 * fm.per_lane} mismatched, worst abs diff {worst}"


@pytest.mark.parametrize("shape", [0, 1])
def test_probe_scattered_by_strided_store_matches_host_matmul(shape):
    """The page's flow end to end on the device: one MFMA, its registers
    scattered into a padded matrix by the library's strided epilogue store, the
    matrix compared with a host matmul; untouched elements stay untouched."""
    fm, mn, k = GEOM[shape]
    rng = np.random.default_rng(200 + shape)
    a = rng.integers(-100, 100, (mn, k)).astype(np.float32)
    b = rng.integers(-100, 100, (k, mn)).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    say("probe + strided store", shape)
    acc = torch.from_numpy(run_probe(shape, "f16", a, b).reshape(-1).copy()).to(device())
    ld, row0, col0 = 3 * mn + 8, 5, mn + 3
    c = torch.full((2 * mn + 7, ld), -7.0, device=device())
    mfl.acc_store_strided(shape, acc, c, row0, col0, ld, stream())
    ch = host(c)
    want = np.full(ch.shape, -7.0)
    want[row0:row0 + mn, col0:col0 + mn] = exact
    assert np.array_equal(ch, want)


@pytest.mark.parametrize("shape", [0, 1])
def test_strided_store_positions(shape):
    fm, mn, _ = GEOM[shape]
    vals = np.arange(64 * fm.per_lane, dtype=np.float32)   # acc[lane*J + j] = lane*J + j
    acc = torch.from_numpy(vals).to(device())
    ld, row0, col0 = 2 * mn + 3, 9, 2
    c = torch.full((row0 + mn + 1, ld), -1.0, device=device())
    say("strided store", shape)
    mfl.acc_store_strided(shape, acc, c, row0, col0, ld, stream())
    flat = host(c).reshape(-1)
    want = np.full(flat.shape, -1.0)
    for l in range(64):
        for j in range(fm.per_lane):
            want[OL.matrix_offset(fm, l, j, row0, col0, ld)] = l * fm.per_lane + j
    assert np.array_equal(flat, want)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_accumulation_rounding(shape, fmt):
    """How one MFMA forms C + sum_k a_k b_k (the explainer warns that
    instruction accumulation may differ from a sequential scalar sum; Strata PR
    #800 describes truncation on another architecture): every probe case must
    give exactly the value of the host model in tests/mfma_sum_model.py — terms
    aligned to the largest one, cut toward zero 26 bits below its top, the sum
    rounded once to fp32, to nearest-even.  Among the cases: 1 + 0.75 ulp rounds
    up; 2^20 + 2^-20 - 2^20 gives 0 (the small product is cut before the
    cancellation); 1 + 0.5 ulp + 2^-40 gives 1 (no sticky bit, a tie to even)."""
    fm, mn, k = GEOM[shape]
    report = {}
    for name, (c00, prods) in MODEL.CASES.items():
        a = np.zeros((mn, k), np.float32)
        b = np.zeros((k, mn), np.float32)
        for i, (x, y) in enumerate(prods):
            a[0, i], b[i, 0] = x, y
        c = np.zeros((mn, mn), np.float32)
        c[0, 0] = c00
        say("accumulation probe", shape, fmt, name)
        acc = run_probe(shape, fmt, a, b, c)
        got = None
        for l in range(64):
            for j in range(fm.per_lane):
                if fm.coords(l, j) == (0, 0):
                    got = float(acc[l, j])
        report[name] = got
        assert got == MODEL.mfma_sum(c00, prods), (name, got, MODEL.mfma_sum(c00, prods))
    print(f"mfma accumulation shape={shape} {fmt}:", report)


# ---- operand fragments through the library (load-side twin of the strided store)

OPNAME = {0: "A", 1: "B"}


def _strided_host(rows, cols, row0, col0, ld, order, outer_pad, rng):
    """A 16-bit matrix (as int16 bits) big enough for a rows x cols tile at
    (row0, col0) in the given order, filled with random bits."""
    outer = (row0 + rows if order == 0 else col0 + cols) + outer_pad
    inner_need = (col0 + cols) if order == 0 else (row0 + rows)
    assert inner_need <= ld
    return rng.integers(-32768, 32768, (outer, ld)).astype(np.int16)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("operand", [0, 1])
@pytest.mark.parametrize("shape", [0, 1])
def test_operand_load_strided_gathers_the_oracle_elements(shape, operand, order):
    """Bit-exact: frag[lane*8 + i] is the matrix element the oracle's operand map
    places at (lane, i), for random origins and leading dimensions."""
    om = OL.OPERAND_MAPS[(shape, OPNAME[operand])]
    rng = np.random.default_rng(300 + 4 * shape + 2 * operand + order)
    for trial in range(3):
        row0, col0 = int(rng.integers(0, 40)), int(rng.integers(0, 40))
        inner = (col0 + om.cols) if order == 0 else (row0 + om.rows)
        ld = inner + int(rng.integers(0, 24))
        m = _strided_host(om.rows, om.cols, row0, col0, ld, order, 3, rng)
        dm = torch.from_numpy(m).to(device())
        frag = torch.empty(64 * 8, dtype=torch.int16, device=device())
        say("operand load", shape, OPNAME[operand], order, row0, col0, ld)
        mfl.operand_load_strided(shape, operand, dm, row0, col0, ld, order, frag, stream())
        got = host(frag).reshape(64, 8)
        flat = m.reshape(-1)
        want = np.array([[flat[OL.operand_matrix_offset(om, l, i, row0, col0, ld, order)] for i in range(8)]
                         for l in range(64)], np.int16)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("orders", [(0, 1), (1, 0), (0, 0), (1, 1)])
@pytest.mark.parametrize("shape", [0, 1])
def test_mma_through_library_layouts_matches_host_matmul(shape, orders, fmt):
    """The whole register-level flow through the exported layouts: A and B tiles
    gathered from strided matrices by operand_load_strided, one raw MFMA, the
    accumulator scattered by acc_store_strided; exact against a host matmul of
    small integers (exact in both 16-bit formats and in fp32)."""
    fm, mn, k = GEOM[shape]
    oa, ob = orders
    rng = np.random.default_rng(400 + shape + 2 * oa + 4 * ob)
    a = rng.integers(-8, 9, (mn, k)).astype(np.float32)
    b = rng.integers(-8, 9, (k, mn)).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64)

    def embed(t, row0, col0, order):
        rows, cols = t.shape
        ld = (col0 + cols if order == 0 else row0 + rows) + 5
        outer = (row0 + rows if order == 0 else col0 + cols) + 2
        big = np.full((outer, ld), np.nan, np.float32)   # NaN outside the tile: any stray read shows
        if order == 0:
            big[row0:row0 + rows, col0:col0 + cols] = t
        else:
            big[col0:col0 + cols, row0:row0 + rows] = t.T
        return big, ld

    abig, lda = embed(a, 3, 9, oa)
    bbig, ldb = embed(b, 6, 2, ob)
    a16, b16 = q16(abig, fmt), q16(bbig, fmt)
    af = torch.empty(512, dtype=torch.int16, device=device())
    bf = torch.empty(512, dtype=torch.int16, device=device())
    acc = torch.full((64 * fm.per_lane,), float("nan"), device=device())
    say("library mma flow", shape, orders, fmt)
    mfl.operand_load_strided(shape, mfl.OPERAND_A, a16, 3, 9, lda, oa, af, stream())
    mfl.operand_load_strided(shape, mfl.OPERAND_B, b16, 6, 2, ldb, ob, bf, stream())
    mfl.mfma_probe(shape, DT[fmt], af, bf, None, acc, stream())
    ldc, row0, col0 = 2 * mn + 5, 4, mn + 1
    c = torch.full((row0 + mn + 2, ldc), -3.0, device=device())
    mfl.acc_store_strided(shape, acc, c, row0, col0, ldc, stream())
    ch = host(c)
    want = np.full(ch.shape, -3.0)
    want[row0:row0 + mn, col0:col0 + mn] = exact
    assert np.array_equal(ch, want)


@pytest.mark.parametrize("fmt,val,scale", [("f16", 2.0 ** -20, 1.0), ("f16", 2.0 ** -24, 1.0),
                                           ("bf16", 2.0 ** -130, 2.0 ** 10), ("bf16", 2.0 ** -133, 2.0 ** 12)])
@pytest.mark.parametrize("shape", [0, 1])
def test_mfma_subnormal_inputs(shape, fmt, val, scale):
    """Subnormal 16-bit operands enter the product unflushed: the lo halves of
    the split (about 2^-11 of a value, so subnormal for small fp16 values) rely
    on it.  Products are chosen to be normal fp32 numbers, compared exactly."""
    fm, mn, k = GEOM[shape]
    a = np.zeros((mn, k), np.float32)
    b = np.zeros((k, mn), np.float32)
    a[3, 5], b[5, 7] = val, scale            # C[3][7] = val * scale
    a[4, 6], b[6, 7] = 3 * val, scale        # C[4][7] = 3 val * scale (3 val still subnormal)
    a[9, 1], a[9, 2], b[1, 2], b[2, 2] = val, val, scale, scale   # C[9][2] = 2 val * scale (a sum)
    from oracle import formats as OF
    assert OF.quantize(np.float32(val), fmt) == val and OF.quantize(np.float32(3 * val), fmt) == 3 * val
    say("mfma subnormal inputs", shape, fmt, val)
    acc = run_probe(shape, fmt, a, b)
    got = np.zeros((mn, mn))
    for l in range(64):
        for j in range(fm.per_lane):
            got[fm.coords(l, j)] = acc[l, j]
    want = np.zeros((mn, mn))
    want[3, 7], want[4, 7], want[9, 2] = val * scale, 3 * val * scale, 2 * val * scale
    assert np.array_equal(got, want), (got[3, 7], got[4, 7], got[9, 2])
