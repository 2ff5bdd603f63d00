"""Pins of the oracle's fp16 / bf16 quantisers and hi/lo split.

The quantiser is written from the value definition of the formats (nearest
multiple of the binade's quantum, ties to even).  It is pinned here against
things other than itself: numpy's float16 conversion and torch's CPU bfloat16
conversion (library routines, both round-to-nearest-even), an independent
nearest-neighbour formulation over all 65,536 bit patterns, and closed forms of
the formats (largest finite value, smallest subnormal, ties)."""
import numpy as np
import pytest
import torch

from oracle import formats as F

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def fp32_from_bits(u):
    return np.asarray(u, dtype=np.uint32).view(np.float32)


def tie_heavy_patterns():
    """fp32 bit patterns that exercise every rounding decision: every upper half
    with the low halves that sit at, just below and just above the bf16 tie, plus
    fp16 values, their neighbours and the fp32 midpoints between consecutive
    fp16 values (and one fp32 ulp either side), plus random patterns."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], np.uint32)
    pats = [(hi[:, None] | lows[None, :]).reshape(-1)]
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    hv = h[np.isfinite(h)].astype(np.float64)
    hv = np.unique(hv)
    mids = ((hv[1:] + hv[:-1]) / 2).astype(np.float32)   # midpoints are exact in fp32
    for base in (hv.astype(np.float32), mids):
        b = base.view(np.uint32)
        pats += [b, b + np.uint32(1), b - np.uint32(1)]
    pats.append(np.random.default_rng(7).integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32))
    return fp32_from_bits(np.concatenate(pats))


@pytest.fixture(scope="module")
def patterns():
    return tie_heavy_patterns()


def same(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(eq | both_nan)


def test_f16_matches_numpy(patterns):
    ours = F.quantize(patterns, "f16")
    lib = patterns.astype(np.float16).astype(np.float64)
    assert same(ours, lib)


def test_bf16_matches_torch(patterns):
    ours = F.quantize(patterns, "bf16")
    lib = torch.from_numpy(patterns.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    assert same(ours, lib)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_matches_nearest_neighbour_formulation(fmt):
    """Independent formulation: decode every finite pattern, sort the values, and
    for each x pick the nearer bracketing value (ties: even bit pattern)."""
    bits = np.arange(1 << 16)
    vals = F.decode_bits(bits, fmt)
    fin = np.isfinite(vals)
    v, b = vals[fin], bits[fin]
    order = np.lexsort((np.signbit(v), v))
    v, b = v[order], b[order]
    # keep one representative per value (+0 and -0 share a value)
    keep = np.concatenate([[True], v[1:] != v[:-1]])
    v, b = v[keep], b[keep]
    rng = np.random.default_rng(11)
    lim = F.FORMATS[fmt][2]
    x = np.concatenate([
        rng.uniform(-lim, lim, 20000),
        rng.standard_normal(20000) * np.exp2(rng.integers(-30, 16, 20000)),
        (v[1:] + v[:-1]) / 2,  # exact ties
    ]).astype(np.float32).astype(np.float64)
    x = x[np.abs(x) <= lim]
    i = np.clip(np.searchsorted(v, x), 1, len(v) - 1)
    lo, hi = v[i - 1], v[i]
    dlo, dhi = x - lo, hi - x
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (b[i] % 2 == 0))
    expect = np.where(pick_hi, hi, lo)
    expect = np.where(x == v[i - 1], lo, expect)
    ours = F.quantize(x, fmt)
    assert np.array_equal(np.abs(ours), np.abs(expect))


def test_closed_forms():
    q16 = lambda x: float(F.quantize(np.float64(x), "f16"))
    qb = lambda x: float(F.quantize(np.float64(x), "bf16"))
    assert q16(65504.0) == 65504.0                   # largest finite fp16
    assert q16(65519.99) == 65504.0                  # below the midpoint to 65536
    assert q16(65520.0) == np.inf                    # tie between 65504 (odd) and 2^16 -> even -> inf
    assert q16(2.0 ** -24) == 2.0 ** -24             # smallest subnormal
    assert q16(2.0 ** -25) == 0.0                    # tie between 0 (even) and 2^-24
    assert q16(3 * 2.0 ** -26) == 2.0 ** -24
    assert q16(1 + 2.0 ** -11) == 1.0                # tie, 1.0 is even
    assert q16(1 + 3 * 2.0 ** -11) == 1 + 2.0 ** -9  # tie, rounds up to the even neighbour
    assert qb(1 + 2.0 ** -8) == 1.0
    assert qb(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert qb(-0.0) == 0.0 and np.signbit(F.quantize(np.float64(-0.0), "bf16"))
    assert int(F.encode_bits(F.quantize(np.float64(1 / 3), "bf16"), "bf16")) == 0x3EAB
    assert int(F.encode_bits(F.quantize(np.float64(1 / 3), "f16"), "f16")) == 0x3555
    assert np.isnan(F.quantize(np.float64(np.nan), "f16"))
    assert F.quantize(np.float64(np.inf), "bf16") == np.inf
    # fp32 max rounds past bf16's largest finite value
    assert qb(float(np.finfo(np.float32).max)) == np.inf


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_bit_codec_roundtrip(fmt):
    bits = np.arange(1 << 16)
    vals = F.decode_bits(bits, fmt)
    ok = ~np.isnan(vals)
    assert np.array_equal(F.encode_bits(vals[ok], fmt), bits[ok])
    assert np.array_equal(F.quantize(vals[ok], fmt), vals[ok])   # representable values are fixed points


def test_bit_codec_known_patterns():
    assert F.decode_bits(0x3C00, "f16") == 1.0
    assert F.decode_bits(0x7BFF, "f16") == 65504.0
    assert F.decode_bits(0x0001, "f16") == 2.0 ** -24
    assert F.decode_bits(0x3F80, "bf16") == 1.0
    assert F.decode_bits(0x7F7F, "bf16") == (2 - 2.0 ** -7) * 2.0 ** 127
    assert F.decode_bits(0xC000, "bf16") == -2.0


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_split_properties(fmt):
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100000) * np.exp2(rng.integers(-6, 6, 100000))).astype(np.float32)
    hi, lo = F.split(x, fmt)
    # hi is the rounded value; lo is the rounded remainder
    assert np.array_equal(hi, F.quantize(x, fmt))
    assert np.array_equal(lo, F.quantize(x.astype(np.float64) - hi, fmt))
    # x - hi is exact in fp32 (the split loses nothing before the second rounding)
    r = x.astype(np.float64) - hi
    assert np.array_equal(r.astype(np.float32).astype(np.float64), r)
    # the two-piece representation error is bounded by half a quantum of lo's binade
    p = F.FORMATS[fmt][0]
    err = np.abs(x - hi - lo)
    bound = np.abs(x) * 2.0 ** (-2 * p + 1) + 2.0 ** -149
    if fmt == "bf16":
        assert np.all(err <= bound)
    # representable inputs split into (x, 0)
    y = F.quantize(x, fmt)
    yh, yl = F.split(y, fmt)
    assert np.array_equal(yh, y) and np.all(yl == 0)
