"""fp64 references for every product the GPU path computes (oracle side).

The tensor-core explainer ("Tensor Core operands: a matrix instruction still
needs a layout contract", paragraph on reference comparisons) separates the
error against the quantised-input problem from the error against the original
problem.  Accordingly:

  * the 16-bit GEMMs (single GEMM, block repeat, dense 4096^3) are compared with
    the fp64 product of the *quantised* operands;
  * the split-precision GEMM is compared with the fp64 product of the
    *original* fp32 operands (its purpose is to recover fp32 accuracy), with the
    exact value of the hi/lo expansion kept as a diagnostic;
  * the attention pair is compared with fp64 attention on the original Q and the
    16-bit K and V (only Q and P are split; K and V are rounded once).

Matrices are passed as the library stores them: A row-major (m x k) and B
column-major, i.e. as Bt = B^T (n x k) row-major.  The fp64 matmul is numpy's
(a library primitive); nothing is blocked, fused or reordered here.
"""
from __future__ import annotations

import numpy as np

from .formats import quantize, split


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def matmul_f64(a, bt) -> np.ndarray:
    """C = A @ B with B given as Bt (B^T), in fp64."""
    return _f64(a) @ _f64(bt).T


def gemm_ref(a, bt, fmt: str) -> np.ndarray:
    """Mixed-precision GEMM on the quantised-input problem: Q(A) @ Q(B) in fp64,
    Q = round-to-nearest-even to ``fmt`` (Warp issue #1965: C accumulated over the
    K loop; the explainer: fp32 accumulation acts on the represented inputs)."""
    return matmul_f64(quantize(a, fmt), quantize(bt, fmt))


def gemm_ref_entries(a, bt, fmt: str, rows, cols) -> np.ndarray:
    """The same values as ``gemm_ref`` at the listed (rows[i], cols[i]) only:
    sum_k Q(A)[r, k] * Q(B)[k, c] in fp64, one dot product per entry."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    qa = quantize(_f64(a)[np.unique(rows)], fmt)
    qb = quantize(_f64(bt)[np.unique(cols)], fmt)
    ra = {r: i for i, r in enumerate(np.unique(rows))}
    cb = {c: i for i, c in enumerate(np.unique(cols))}
    return np.array([np.dot(qa[ra[r]], qb[cb[c]]) for r, c in zip(rows, cols)])


def block_repeat_ref(a, bt, tk: int, repeats: int, fmt: str) -> np.ndarray:
    """Block-repeat spike (Warp issue #1965, "Spike" section): every workgroup
    loads one A tile (its TM rows, K columns 0..TK-1) and one B tile (its TN
    columns, K rows 0..TK-1) once and accumulates ``repeats`` block products into
    the same accumulator, so each output tile equals repeats * A_tile @ B_tile,
    and over the whole output C = repeats * Q(A[:, :TK]) @ Q(B[:TK, :])."""
    return float(repeats) * matmul_f64(quantize(_f64(a)[:, :tk], fmt),
                                       quantize(_f64(bt)[:, :tk], fmt))


def split_ref(a, bt) -> np.ndarray:
    """Acceptance reference of the split-precision GEMM: A @ B in fp64 on the
    original fp32 values (the original-problem error of the explainer)."""
    return matmul_f64(a, bt)


def split_expansion(a, bt, fmt: str, split_a: bool = True, split_b: bool = True,
                    lolo: bool = False) -> np.ndarray:
    """Exact (fp64) value of what the split algorithm sums (Strata PR #800, "What's
    going on" and "The fix"): each split operand is x = hi + lo with
    hi = Q(x), lo = Q(x - hi); an operand that is not split is rounded once,
    Q(x).  The expansion is hi_a.hi_b + hi_a.lo_b + lo_a.hi_b (+ lo_a.lo_b),
    dropping the terms of an unsplit operand's (absent) lo part."""
    if split_a:
        ah, al = split(a, fmt)
    else:
        ah, al = quantize(a, fmt), None
    if split_b:
        bh, bl = split(bt, fmt)
    else:
        bh, bl = quantize(bt, fmt), None
    r = matmul_f64(ah, bh)
    if bl is not None:
        r = r + matmul_f64(ah, bl)
    if al is not None:
        r = r + matmul_f64(al, bh)
    if lolo and al is not None and bl is not None:
        r = r + matmul_f64(al, bl)
    return r


def softmax_rows(s):
    """Row softmax pieces in fp64: m = max_k S, P~ = exp(S - m), l = sum_k P~.
    softmax(S) = P~ / l.  (Strata PR #800 applies the softmax between the two
    GEMMs; the split variant divides by l after the second GEMM.)"""
    s = _f64(s)
    m = s.max(axis=1, keepdims=True)
    pt = np.exp(s - m)
    return pt, m[:, 0], pt.sum(axis=1)


def attention_ref(q, k, v, fmt: str = "f16", round_kv: bool = True) -> np.ndarray:
    """O = softmax(Q @ Q16(K)^T) @ Q16(V) in fp64, with Q at its original fp32
    values and K, V rounded once to ``fmt`` (Strata PR #800: only q and p are
    split; the pages state neither a causal mask nor a 1/sqrt(d) scale, so there
    is none).  round_kv=False keeps K and V at their original fp32 values too:
    the reference of the variant that splits K and V as well, where every
    operand is carried at fp32-input accuracy."""
    kk = quantize(k, fmt) if round_kv else _f64(k)
    vv = quantize(v, fmt) if round_kv else _f64(v)
    s = matmul_f64(q, kk)
    pt, _, l = softmax_rows(s)
    return (pt / l[:, None]) @ vv


def rel_error(c, r) -> float:
    """Normwise relative error ||C - R||_F / ||R||_F in fp64 (the pages report a
    relative error against an fp64 reference without naming the norm; the
    Frobenius norm is the reading taken)."""
    c = _f64(c)
    r = _f64(r)
    return float(np.linalg.norm(c - r) / np.linalg.norm(r))
