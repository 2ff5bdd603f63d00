"""Accumulator-fragment layouts, enumerated by brute force (oracle side).

cuda-oxide PR #474 ("derive the m16n8k16 accumulator fragment layout") treats a
warp-level MMA's accumulator as a map (lane, j) -> (row, col) over the output
tile and checks it is a bijection "via an ownership map" that fails on both
overlap and gap ("Tests" section).  This module does exactly that, with plain
loops over every point, for any map given in row/col form:

  * the page's own worked example, NVIDIA m16n8k16 (32 lanes x 4 values, 16x8),
    used to pin the machinery to the numbers the page prints ("The layout is a
    mixed-radix numeral" section);
  * the two AMD CDNA4 accumulator layouts this library targets,
    V_MFMA_F32_16X16X32_{F16,BF16} (64 lanes x 4 values, 16x16) and
    V_MFMA_F32_32X32X16_{F16,BF16} (64 lanes x 16 values, 32x32), written in
    row/col form from the CDNA matrix-core output layout.  These two maps are
    pinned by the bijection check here and, on the device, by raw MFMA probes
    whose registers name their own coordinates; they have no printed values in
    the pages (parity for them rests on the hardware probe).

The same machinery covers the operand fragments of those two instructions
(which lane supplies which element of A and B), the half of the layout contract
the cuda-oxide page leaves out of scope ("Scope" section).  Operand maps are
pinned like the accumulator maps: bijection here, hardware on the device (a raw
MFMA fed through these maps must reproduce a host matmul exactly).

The inverse map (decode) is built here by inverting the enumeration, never by a
closed formula, so that it is independent of the library's numeral arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Dict, List, Optional, Tuple

INT64_MAX = (1 << 63) - 1


@dataclass(frozen=True)
class FragmentMap:
    name: str
    lanes: int          # lanes of the wave (or warp) that hold the tile
    per_lane: int       # accumulator values per lane (J)
    rows: int
    cols: int
    coords: Callable[[int, int], Tuple[int, int]]   # (lane, j) -> (row, col)


# cuda-oxide PR #474: group = lane / 4, tig = lane % 4,
# row = group + 8*(j >> 1), col = 2*tig + (j & 1)  (the page's worked example).
M16N8K16 = FragmentMap(
    "m16n8k16", 32, 4, 16, 8,
    lambda lane, j: (lane // 4 + 8 * (j >> 1), 2 * (lane % 4) + (j & 1)),
)

# CDNA4 V_MFMA_F32_16X16X32_{F16,BF16}: lane l holds column l mod 16 and the
# four consecutive rows 4*(l div 16) .. 4*(l div 16)+3 (value j is row +j).
MFMA_16X16X32 = FragmentMap(
    "mfma_16x16x32", 64, 4, 16, 16,
    lambda lane, j: (4 * (lane // 16) + j, lane % 16),
)

# CDNA4 V_MFMA_F32_32X32X16_{F16,BF16}: lane l holds column l mod 32; its 16
# values are four groups of four consecutive rows; group g = j div 4 starts at
# row 8*g + 4*(l div 32).
MFMA_32X32X16 = FragmentMap(
    "mfma_32x32x16", 64, 16, 32, 32,
    lambda lane, j: (8 * (j // 4) + 4 * (lane // 32) + (j % 4), lane % 32),
)

MAPS = {m.name: m for m in (M16N8K16, MFMA_16X16X32, MFMA_32X32X16)}


# ---- operand fragments of the CDNA4 f16/bf16 MFMA instructions
#
# Each lane supplies 8 consecutive K positions of one row of A (MN x K) and of
# one column of B (K x MN): lane l holds A[l mod MN][8*(l div MN) + i] and
# B[8*(l div MN) + i][l mod MN], i = 0..7.  With 64 lanes, 16x16x32 has four
# K groups of 8 (K = 32) and 32x32x16 has two (K = 16).  coords are (row, col)
# of the operand as written: (m, k) for A, (k, n) for B.

@dataclass(frozen=True)
class OperandMap:
    name: str
    operand: str        # "A" or "B"
    lanes: int
    per_lane: int       # 16-bit elements per lane (8: one 16-byte register group)
    rows: int           # A: MN, B: K
    cols: int           # A: K,  B: MN
    coords: Callable[[int, int], Tuple[int, int]]   # (lane, i) -> (row, col)


def _operand_map(name: str, operand: str, mn: int, k: int) -> OperandMap:
    if operand == "A":
        return OperandMap(name, "A", 64, 8, mn, k, lambda lane, i: (lane % mn, 8 * (lane // mn) + i))
    return OperandMap(name, "B", 64, 8, k, mn, lambda lane, i: (8 * (lane // mn) + i, lane % mn))


OPERAND_MAPS = {
    (0, "A"): _operand_map("mfma_16x16x32.A", "A", 16, 32),
    (0, "B"): _operand_map("mfma_16x16x32.B", "B", 16, 32),
    (1, "A"): _operand_map("mfma_32x32x16.A", "A", 32, 16),
    (1, "B"): _operand_map("mfma_32x32x16.B", "B", 32, 16),
}


def operand_offset(om: OperandMap, lane: int, i: int) -> int:
    """Offset of (lane, i) in the K-contiguous storage of the operand tile:
    A row-major (m*K + k), B column-major (n*K + k)."""
    r, c = om.coords(lane, i)
    return r * om.cols + c if om.operand == "A" else c * om.rows + r


def operand_decode_table(om: OperandMap) -> Dict[int, Tuple[int, int]]:
    """Inverse of ``operand_offset`` by enumeration; raises on a shared offset."""
    inv: Dict[int, Tuple[int, int]] = {}
    for lane in range(om.lanes):
        for i in range(om.per_lane):
            o = operand_offset(om, lane, i)
            if o in inv:
                raise ValueError(f"{om.name}: offset {o} owned twice")
            inv[o] = (lane, i)
    return inv


def operand_is_bijection(om: OperandMap) -> bool:
    """Every (row, col) of the operand tile supplied by exactly one (lane, i)."""
    if om.lanes * om.per_lane != om.rows * om.cols:
        return False
    own = [[0] * om.cols for _ in range(om.rows)]
    for lane in range(om.lanes):
        for i in range(om.per_lane):
            r, c = om.coords(lane, i)
            if not (0 <= r < om.rows and 0 <= c < om.cols):
                return False
            own[r][c] += 1
    return all(v == 1 for row in own for v in row)


def operand_matrix_offset(om: OperandMap, lane: int, i: int, row0: int, col0: int, ld: int,
                          order: int) -> Optional[int]:
    """Element offset of (lane, i) when the operand tile's origin sits at
    (row0, col0) of a matrix with leading dimension ``ld``: row-major (order 0)
    (row0+row)*ld + col0+col, column-major (order 1) (col0+col)*ld + row0+row.
    None on overflow: the contiguous coordinate reaches ``ld`` (it would spill
    into the next row or column) or the value does not fit a signed 64-bit
    offset — the reading taken for the accumulator's strided destination."""
    if row0 < 0 or col0 < 0 or ld <= 0 or order not in (0, 1):
        raise ValueError("negative origin, non-positive leading dimension or bad order")
    r, c = om.coords(lane, i)
    outer, inner = (row0 + r, col0 + c) if order == 0 else (col0 + c, row0 + r)
    if inner >= ld:
        return None
    out = outer * ld + inner
    return None if out > INT64_MAX else out


def ownership(fm: FragmentMap) -> List[List[int]]:
    """Count, for every (row, col) of the tile, how many (lane, j) land on it.
    Points outside the tile raise."""
    own = [[0] * fm.cols for _ in range(fm.rows)]
    for lane in range(fm.lanes):
        for j in range(fm.per_lane):
            r, c = fm.coords(lane, j)
            if not (0 <= r < fm.rows and 0 <= c < fm.cols):
                raise ValueError(f"{fm.name}: ({lane},{j}) -> ({r},{c}) outside the tile")
            own[r][c] += 1
    return own


def is_bijection(fm: FragmentMap) -> bool:
    """True iff every tile position is owned exactly once (no overlap, no gap)."""
    if fm.lanes * fm.per_lane != fm.rows * fm.cols:
        return False
    try:
        own = ownership(fm)
    except ValueError:
        return False
    return all(v == 1 for row in own for v in row)


def offset(fm: FragmentMap, lane: int, j: int) -> int:
    """Row-major offset of (lane, j) inside the tile: row * cols + col."""
    r, c = fm.coords(lane, j)
    return r * fm.cols + c


def offset_table(fm: FragmentMap) -> List[List[int]]:
    """offset(lane, j) for every lane and j."""
    return [[offset(fm, lane, j) for j in range(fm.per_lane)] for lane in range(fm.lanes)]


def decode_table(fm: FragmentMap) -> Dict[int, Tuple[int, int]]:
    """Inverse of ``offset`` by enumeration: offset -> (lane, j).  Raises if two
    points share an offset."""
    inv: Dict[int, Tuple[int, int]] = {}
    for lane in range(fm.lanes):
        for j in range(fm.per_lane):
            o = offset(fm, lane, j)
            if o in inv:
                raise ValueError(f"{fm.name}: offset {o} owned twice")
            inv[o] = (lane, j)
    return inv


def matrix_offset(fm: FragmentMap, lane: int, j: int, row0: int, col0: int,
                  ld: int) -> Optional[int]:
    """Element offset of (lane, j) when the tile's origin sits at (row0, col0) of a
    row-major matrix with leading dimension ``ld``: (row0+row)*ld + col0+col.

    cuda-oxide PR #474, "API": the strided destination a GEMM epilogue writes,
    None on overflow.  Reading of "overflow" (the page does not define it): the
    value does not fit a signed 64-bit offset, or the column col0+col reaches
    ``ld`` and would spill into the next row.  Negative origins or ``ld`` are
    rejected with ValueError.  Python integers are unbounded, so the check is
    exact."""
    if row0 < 0 or col0 < 0 or ld <= 0:
        raise ValueError("negative origin or non-positive leading dimension")
    r, c = fm.coords(lane, j)
    if col0 + c >= ld:
        return None
    out = (row0 + r) * ld + (col0 + c)
    if out > INT64_MAX:
        return None
    return out


# ---- the mixed-radix numeral (cuda-oxide PR #474, "The layout is a mixed-radix numeral")

@dataclass(frozen=True)
class Digit:
    name: str
    radix: int


def place_values(digits: List[Digit]) -> List[int]:
    """Place value of each digit: the running product of the lower radices."""
    places, p = [], 1
    for d in digits:
        places.append(p)
        p *= d.radix
    return places


def span(digits: List[Digit]) -> int:
    """Number of distinct values of the numeral: the product of all radices."""
    s = 1
    for d in digits:
        s *= d.radix
    return s


def numeral_value(digits: List[Digit], values: Dict[str, int]) -> int:
    """sum(digit value * place value); each digit value must lie in [0, radix)."""
    total = 0
    for d, p in zip(digits, place_values(digits)):
        v = values[d.name]
        if not 0 <= v < d.radix:
            raise ValueError(f"digit {d.name}={v} outside [0,{d.radix})")
        total += v * p
    return total


# The page's digit table for m16n8k16, lowest place first.
M16N8K16_DIGITS = [Digit("j&1", 2), Digit("tig", 4), Digit("group", 8), Digit("j>>1", 2)]


def m16n8k16_digit_values(lane: int, j: int) -> Dict[str, int]:
    return {"j&1": j & 1, "tig": lane % 4, "group": lane // 4, "j>>1": j >> 1}
