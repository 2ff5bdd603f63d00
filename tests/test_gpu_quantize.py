"""Device rounding and hi/lo splitting against the oracle's quantiser, bit for
bit, on tie-heavy fp32 patterns and ragged lengths."""
import numpy as np
import pytest
import torch

import mma_fragment_layouts_amd as mfl
from oracle import formats as F

from _gpu import DT, dev32, device, host, say, stream

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def patterns(n_random=1 << 20):
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1000, 0xF000], np.uint32)
    p = [(hi[:, None] | lows[None, :]).reshape(-1)]
    p.append(np.random.default_rng(1).integers(0, 1 << 32, n_random, dtype=np.uint64).astype(np.uint32))
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    h = np.unique(h[np.isfinite(h)])
    mids = ((h[1:] + h[:-1]) / 2).astype(np.float32).view(np.uint32)
    p += [mids, mids + np.uint32(1), mids - np.uint32(1)]
    return np.concatenate(p).view(np.float32)


def bits_equal(dev_bits, want_vals, fmt):
    got = dev_bits.astype(np.int64) & 0xFFFF
    want = F.encode_bits(want_vals, fmt)
    nan = np.isnan(want_vals)
    # NaN: any NaN pattern is acceptable; everything else bit-exact
    got_nan = np.isnan(F.decode_bits(got, fmt))
    return bool(np.all(np.where(nan, got_nan, got == want)))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_quantize_bit_exact(fmt):
    x = patterns()
    say("quantize", fmt, x.size)
    src = dev32(x)
    out = torch.empty(x.size, dtype=torch.int16, device=device())
    mfl.quantize_fp32(DT[fmt], src, out, x.size, stream())
    assert bits_equal(host(out), F.quantize(x, fmt), fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_split_bit_exact(fmt):
    rng = np.random.default_rng(2)
    x = np.concatenate([
        (rng.standard_normal(300000) * np.exp2(rng.integers(-20, 20, 300000))).astype(np.float32),
        patterns(1 << 16)[::7],
    ])
    x = x[np.abs(x) < 6e4] if fmt == "f16" else x
    say("split", fmt, x.size)
    src = dev32(x)
    hi = torch.empty(x.size, dtype=torch.int16, device=device())
    lo = torch.empty(x.size, dtype=torch.int16, device=device())
    mfl.split_fp32(DT[fmt], src, hi, lo, x.size, stream())
    whi, wlo = F.split(x, fmt)
    assert bits_equal(host(hi), whi, fmt)
    assert bits_equal(host(lo), wlo, fmt)


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1023, 4097])
def test_ragged_lengths_do_not_touch_past_n(n):
    x = np.random.default_rng(n).standard_normal(n).astype(np.float32)
    say("ragged quantize", n)
    src = dev32(x)
    out = torch.full((n + 16,), 0x5A5A, dtype=torch.int16, device=device())
    mfl.quantize_fp32(mfl.BF16, src, out, n, stream())
    h = host(out)
    assert bits_equal(h[:n], F.quantize(x, "bf16"), "bf16")
    assert np.all(h[n:] == 0x5A5A)
