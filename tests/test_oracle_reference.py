"""Pins of the oracle's fp64 references: brute force on tiny inputs, exact
integer-valued products, closed forms (all-ones, identity, repeat factor,
uniform softmax), and special cases of attention."""
import math

import numpy as np
import pytest

from oracle import formats as F
from oracle import reference as R


def brute_matmul(a, bt):
    m, k = a.shape
    n = bt.shape[0]
    return np.array([[sum(float(a[i, t]) * float(bt[j, t]) for t in range(k)) for j in range(n)]
                     for i in range(m)])


def test_matmul_brute_force_asymmetric():
    rng = np.random.default_rng(0)
    a = rng.integers(-50, 50, (5, 7)).astype(np.float32)
    bt = rng.integers(-50, 50, (3, 7)).astype(np.float32)
    assert np.array_equal(R.matmul_f64(a, bt), brute_matmul(a, bt))
    # a transposed operand is a different product
    assert not np.array_equal(R.matmul_f64(a, bt).T[:3, :3], brute_matmul(a, bt)[:3, :3])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_gemm_ref_exact_on_integers(fmt):
    rng = np.random.default_rng(1)
    a = rng.integers(-128, 128, (9, 33)).astype(np.float32)
    bt = rng.integers(-128, 128, (11, 33)).astype(np.float32)
    exact = np.array([[sum(int(a[i, t]) * int(bt[j, t]) for t in range(33)) for j in range(11)]
                      for i in range(9)], dtype=np.float64)
    assert np.array_equal(R.gemm_ref(a, bt, fmt), exact)


def test_gemm_ref_quantises_inputs():
    a = np.full((2, 3), 1 + 2.0 ** -9, np.float32)      # not a bf16 value: rounds to 1
    bt = np.ones((2, 3), np.float32)
    assert np.all(R.gemm_ref(a, bt, "bf16") == 3.0)
    assert np.all(R.gemm_ref(a, bt, "f16") == 3 * (1 + 2.0 ** -9))   # exact in fp16


def test_gemm_ref_closed_forms():
    k = 64
    ones = np.ones((8, k), np.float32)
    assert np.all(R.gemm_ref(ones, ones, "bf16") == k)
    rng = np.random.default_rng(2)
    x = rng.uniform(-1, 1, (16, 16)).astype(np.float32)
    eye = np.eye(16, dtype=np.float32)
    assert np.array_equal(R.gemm_ref(x, eye, "f16"), F.quantize(x, "f16"))
    assert np.array_equal(R.gemm_ref(eye, x, "f16"), F.quantize(x, "f16").T)


def test_gemm_ref_entries_match_full():
    rng = np.random.default_rng(3)
    a = rng.uniform(-1, 1, (40, 24)).astype(np.float32)
    bt = rng.uniform(-1, 1, (30, 24)).astype(np.float32)
    full = R.gemm_ref(a, bt, "bf16")
    rows = rng.integers(0, 40, 50)
    cols = rng.integers(0, 30, 50)
    assert np.allclose(R.gemm_ref_entries(a, bt, "bf16", rows, cols), full[rows, cols], rtol=0, atol=1e-12)


def test_block_repeat_brute_force():
    rng = np.random.default_rng(4)
    tm, tn, tk, reps = 4, 3, 5, 7
    a = rng.integers(-8, 8, (2 * tm, tk)).astype(np.float32)
    bt = rng.integers(-8, 8, (3 * tn, tk)).astype(np.float32)
    out = np.zeros((2 * tm, 3 * tn))
    for bi in range(2):
        for bj in range(3):
            at = a[bi * tm:(bi + 1) * tm]
            btt = bt[bj * tn:(bj + 1) * tn]
            acc = np.zeros((tm, tn))
            for _ in range(reps):
                acc = acc + brute_matmul(at, btt)
            out[bi * tm:(bi + 1) * tm, bj * tn:(bj + 1) * tn] = acc
    assert np.array_equal(R.block_repeat_ref(a, bt, tk, reps, "f16"), out)
    # only the first tk columns take part
    wide = np.concatenate([a, np.full((2 * tm, 3), np.nan, np.float32)], axis=1)
    wide_b = np.concatenate([bt, np.full((3 * tn, 3), np.nan, np.float32)], axis=1)
    assert np.array_equal(R.block_repeat_ref(wide, wide_b, tk, reps, "f16"), out)


def test_split_expansion_exact_cases():
    rng = np.random.default_rng(5)
    # values that are exactly hi + lo with both pieces bf16: expansion with lo.lo is exact
    hi = F.quantize(rng.standard_normal((6, 10)), "bf16")
    lo = F.quantize(hi * rng.uniform(-2 ** -9, 2 ** -9, hi.shape), "bf16")
    x = (hi + lo).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), hi + lo)
    hb = F.quantize(rng.standard_normal((7, 10)), "bf16")
    lb = F.quantize(hb * rng.uniform(-2 ** -9, 2 ** -9, hb.shape), "bf16")
    y = (hb + lb).astype(np.float32)
    exact = R.split_ref(x, y)
    assert np.allclose(R.split_expansion(x, y, "bf16", lolo=True), exact, rtol=1e-14, atol=0)
    # without lo.lo the missing term is exactly lo_a . lo_b
    diff = exact - R.split_expansion(x, y, "bf16")
    assert np.allclose(diff, lo @ lb.T, rtol=1e-10, atol=1e-300)
    # an unsplit operand contributes only its rounded value
    assert np.array_equal(R.split_expansion(x, y, "bf16", split_b=False),
                          R.matmul_f64(hi, hb) + R.matmul_f64(lo, hb))


def test_split_expansion_error_shrinks_with_more_terms():
    rng = np.random.default_rng(6)
    a = rng.standard_normal((64, 512)).astype(np.float32)
    bt = rng.standard_normal((64, 512)).astype(np.float32)
    ref = R.split_ref(a, bt)
    e1 = R.rel_error(R.gemm_ref(a, bt, "bf16"), ref)
    e3 = R.rel_error(R.split_expansion(a, bt, "bf16"), ref)
    e4 = R.rel_error(R.split_expansion(a, bt, "bf16", lolo=True), ref)
    assert e4 < e3 < e1
    assert 1e-6 < e3 < 2e-5     # ~16 significant bits: far below bf16, above fp32
    assert e1 > 1e-3


def test_softmax_closed_forms():
    s = np.array([[0.0, math.log(2.0)], [5.0, 5.0]])
    pt, m, l = R.softmax_rows(s)
    p = pt / l[:, None]
    assert np.allclose(p, [[1 / 3, 2 / 3], [0.5, 0.5]], rtol=1e-15)
    assert np.array_equal(m, [math.log(2.0), 5.0])
    assert np.all(pt <= 1.0) and np.all(pt.max(axis=1) == 1.0)
    # shift invariance
    pt2, _, l2 = R.softmax_rows(s + 100.0)
    assert np.allclose(pt2 / l2[:, None], p, rtol=1e-14)


def test_attention_special_cases():
    rng = np.random.default_rng(7)
    nk, d = 64, 8
    k = rng.standard_normal((nk, d)).astype(np.float32)
    v = rng.standard_normal((nk, d)).astype(np.float32)
    # Q = 0 -> uniform probabilities -> column means of Q16(V)
    o = R.attention_ref(np.zeros((3, d), np.float32), k, v)
    assert np.allclose(o, np.tile(F.quantize(v, "f16").mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-15)
    # one overwhelming score picks that row of Q16(V)
    q = (F.quantize(k[5], "f16") * 400.0)[None, :].astype(np.float32)
    o = R.attention_ref(q, k, v)
    assert np.allclose(o[0], F.quantize(v[5], "f16"), atol=1e-10)
    # V = one-hot columns -> O = P
    q = rng.standard_normal((4, d)).astype(np.float32)
    kk = rng.standard_normal((d, d)).astype(np.float32)
    o = R.attention_ref(q, kk, np.eye(d, dtype=np.float32))
    s = q.astype(np.float64) @ F.quantize(kk, "f16").T
    p = np.exp(s - s.max(axis=1, keepdims=True))
    assert np.allclose(o, p / p.sum(axis=1, keepdims=True), rtol=1e-13)


def test_attention_brute_force_tiny():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((2, 3)).astype(np.float32)
    k = rng.standard_normal((4, 3)).astype(np.float32)
    v = rng.standard_normal((4, 3)).astype(np.float32)
    kq, vq = F.quantize(k, "f16"), F.quantize(v, "f16")
    out = np.zeros((2, 3))
    for i in range(2):
        s = [sum(float(q[i, t]) * kq[j, t] for t in range(3)) for j in range(4)]
        w = [math.exp(x) for x in s]
        tot = sum(w)
        for c in range(3):
            out[i, c] = sum(w[j] / tot * vq[j, c] for j in range(4))
    assert np.allclose(R.attention_ref(q, k, v), out, rtol=1e-13)


def test_attention_unrounded_kv():
    """round_kv=False: K and V enter at their fp32 values.  Pinned by (1) equality
    with the rounded reference when K and V are exactly representable in fp16,
    (2) the Q = 0 closed form (column means of V itself), (3) brute force."""
    rng = np.random.default_rng(9)
    nk, d = 48, 8
    k16 = F.quantize(rng.standard_normal((nk, d)).astype(np.float32), "f16").astype(np.float32)
    v16 = F.quantize(rng.standard_normal((nk, d)).astype(np.float32), "f16").astype(np.float32)
    q = rng.standard_normal((5, d)).astype(np.float32)
    assert np.array_equal(R.attention_ref(q, k16, v16, round_kv=False), R.attention_ref(q, k16, v16))
    v = (rng.standard_normal((nk, d)) * (1 + 2.0 ** -13)).astype(np.float32)   # not fp16-representable
    o = R.attention_ref(np.zeros((2, d), np.float32), k16, v, round_kv=False)
    assert np.allclose(o, np.tile(v.astype(np.float64).mean(axis=0), (2, 1)), rtol=1e-13, atol=1e-15)
    assert not np.allclose(o, R.attention_ref(np.zeros((2, d), np.float32), k16, v), rtol=1e-9, atol=0)
    k = rng.standard_normal((3, 2)).astype(np.float32)
    vv = rng.standard_normal((3, 2)).astype(np.float32)
    qq = rng.standard_normal((1, 2)).astype(np.float32)
    w = [math.exp(float(qq[0, 0]) * float(k[j, 0]) + float(qq[0, 1]) * float(k[j, 1])) for j in range(3)]
    out = [sum(w[j] * float(vv[j, c]) for j in range(3)) / sum(w) for c in range(2)]
    assert np.allclose(R.attention_ref(qq, k, vv, round_kv=False)[0], out, rtol=1e-13)


def test_rel_error_closed_form():
    r = np.arange(1, 10, dtype=np.float64).reshape(3, 3)
    assert math.isclose(R.rel_error(r * (1 + 1e-6), r), 1e-6, rel_tol=1e-9)
    assert R.rel_error(r, r) == 0.0
