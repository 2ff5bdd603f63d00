"""16-bit floating-point formats, written from their definitions (oracle side).

The tensor-core explainer ("Tensor Core operands: a matrix instruction still
needs a layout contract", paragraph on mixed precision) says that converting to
FP16 changes the values entering the multiply and that FP16 and BF16 are
different error models.  Neither page states a rounding mode; the reading taken
here is IEEE 754 round-to-nearest, ties-to-even (the IEEE default).

Both formats are described by (precision p, minimum normal exponent emin,
maximum finite value); a finite value is quantised by choosing the quantum of
its binade (or of the subnormal range) and rounding to the nearest multiple of
it, ties to an even multiple.  All arithmetic is in fp64, where every fp32 value
and every quotient by a power of two is exact.
"""
from __future__ import annotations

import numpy as np

# (precision in bits including the implicit one, emin, max finite value)
FORMATS = {
    # IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
    "f16": (11, -14, (2.0 - 2.0 ** -10) * 2.0 ** 15),
    # bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
    "bf16": (8, -126, (2.0 - 2.0 ** -7) * 2.0 ** 127),
}


def quantize(x, fmt: str) -> np.ndarray:
    """Round each element of ``x`` (fp32 or fp64 values) to the nearest value of
    ``fmt`` ('f16' or 'bf16'), ties to even; overflow goes to +-inf, NaN stays
    NaN, signed zeros keep their sign, subnormals are produced gradually.
    Returns fp64 values (each exactly representable in ``fmt``)."""
    p, emin, fmax = FORMATS[fmt]
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    finite = np.isfinite(x) & (x != 0)
    ax = np.abs(x[finite])
    # binade exponent: |x| = m * 2**e2 with m in [0.5, 1)  ->  floor(log2|x|) = e2 - 1
    _, e2 = np.frexp(ax)
    e = np.maximum(e2 - 1, emin)               # below emin the subnormal quantum applies
    quantum = np.ldexp(1.0, e - (p - 1))
    r = np.rint(ax / quantum) * quantum        # np.rint rounds half to even
    r = np.where(r > fmax, np.inf, r)          # rounding past the largest finite value
    out[finite] = np.copysign(r, x[finite])
    return out


def split(x, fmt: str):
    """hi/lo split of fp32 values (Strata PR #800, "What's going on": q and p are
    split into an FP16 hi half and a lo half): hi = Q(x), lo = Q(x - hi), with
    x - hi formed exactly in fp64.  Returns (hi, lo) as fp64 arrays."""
    x = np.asarray(x, dtype=np.float64)
    hi = quantize(x, fmt)
    with np.errstate(invalid="ignore"):
        lo = quantize(x - hi, fmt)
    return hi, lo


# ---- bit-pattern views, used by the tests to compare with device bit patterns ----

def decode_bits(bits, fmt: str) -> np.ndarray:
    """Value of 16-bit patterns under ``fmt``, from the field definitions:
    sign s, biased exponent E, fraction F; normal (-1)^s 2^(E-bias) (1 + F/2^f),
    subnormal (-1)^s 2^(1-bias) F/2^f, E all-ones -> inf (F=0) or NaN."""
    p, emin, _ = FORMATS[fmt]
    fbits = p - 1
    ebits = 15 - fbits
    bias = (1 << (ebits - 1)) - 1
    b = np.asarray(bits, dtype=np.int64) & 0xFFFF
    s = (b >> 15) & 1
    E = (b >> fbits) & ((1 << ebits) - 1)
    F = b & ((1 << fbits) - 1)
    sign = np.where(s == 1, -1.0, 1.0)
    normal = np.ldexp(1.0 + F / float(1 << fbits), (E - bias).astype(np.int64))
    sub = np.ldexp(F / float(1 << fbits), 1 - bias)
    val = np.where(E == 0, sub, normal)
    val = np.where(E == (1 << ebits) - 1, np.where(F == 0, np.inf, np.nan), val)
    return sign * val


def encode_bits(v, fmt: str) -> np.ndarray:
    """16-bit pattern of values already representable in ``fmt`` (the inverse of
    ``decode_bits`` on non-NaN values; NaN maps to the canonical quiet NaN)."""
    p, emin, _ = FORMATS[fmt]
    fbits = p - 1
    ebits = 15 - fbits
    bias = (1 << (ebits - 1)) - 1
    v = np.asarray(v, dtype=np.float64)
    s = np.signbit(v).astype(np.int64)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.int64)
    isnan = np.isnan(v)
    isinf = np.isinf(v)
    fin = ~isnan & ~isinf & (a > 0)
    _, e2 = np.frexp(a[fin])
    e = e2 - 1
    normal = e >= emin
    E = np.where(normal, e + bias, 0)
    F = np.where(normal, np.ldexp(a[fin], -e) - 1.0, np.ldexp(a[fin], -emin)) * (1 << fbits)
    if not np.all(F == np.rint(F)):
        raise ValueError("value not representable in " + fmt)
    out[fin] = (E.astype(np.int64) << fbits) | F.astype(np.int64)
    out[isinf] = ((1 << ebits) - 1) << fbits
    out[isnan] = (((1 << ebits) - 1) << fbits) | (1 << (fbits - 1))
    return (out | (s << 15)) & 0xFFFF
