"""Pins of the oracle's fragment-layout enumerator.

The enumerator is pinned to the worked example the cuda-oxide page prints
(m16n8k16 digit table, span, the split fragment index) read from
tests/golden/p1_m16n8k16_numeral.txt, and to planted mistakes: a dropped term,
a swapped index or a transposed map must each be caught by one of the checks.
The two CDNA4 maps are checked as bijections here; their device agreement is
the GPU probe test's job."""
import os

import numpy as np
import pytest

from oracle import layouts as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "p1_m16n8k16_numeral.txt")


def read_golden():
    digits, kv, steps = [], {}, {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            t = line.split()
            if t[0] == "digit":
                digits.append((t[1], int(t[2]), int(t[3])))
            elif t[0] == "step":
                steps[t[1]] = (int(t[3]), int(t[5]))
            else:
                kv[t[0]] = int(t[1])
    return digits, kv, steps


def test_worked_example_digit_table():
    digits, kv, _ = read_golden()
    assert [(d.name, d.radix) for d in L.M16N8K16_DIGITS] == [(n, r) for n, r, _ in digits]
    assert L.place_values(L.M16N8K16_DIGITS) == [p for _, _, p in digits]
    assert L.span(L.M16N8K16_DIGITS) == kv["span"]
    fm = L.M16N8K16
    assert (fm.rows, fm.cols, fm.lanes, fm.per_lane) == (kv["tile_rows"], kv["tile_cols"], kv["lanes"], kv["per_lane"])


def test_worked_example_numeral_equals_rowmajor_offset():
    fm = L.M16N8K16
    for lane in range(32):
        for j in range(4):
            assert L.numeral_value(L.M16N8K16_DIGITS, L.m16n8k16_digit_values(lane, j)) == L.offset(fm, lane, j)


def test_worked_example_bijection_and_inverse():
    fm = L.M16N8K16
    assert L.is_bijection(fm)
    inv = L.decode_table(fm)
    assert sorted(inv) == list(range(128))
    for lane in range(32):
        for j in range(4):
            assert inv[L.offset(fm, lane, j)] == (lane, j)


def test_worked_example_split_fragment_index():
    _, _, steps = read_golden()
    fm = L.M16N8K16
    for lane in range(32):
        r0, c0 = fm.coords(lane, 0)
        r1, c1 = fm.coords(lane, 1)
        r2, c2 = fm.coords(lane, 2)
        assert (r1 - r0, c1 - c0) == steps["j0_j1"]
        assert (r2 - r0, c2 - c0) == steps["j0_j2"]


@pytest.mark.parametrize("name,npts", [("mfma_16x16x32", 256), ("mfma_32x32x16", 1024)])
def test_cdna4_maps_are_bijections(name, npts):
    fm = L.MAPS[name]
    assert fm.lanes * fm.per_lane == npts == fm.rows * fm.cols
    assert L.is_bijection(fm)
    inv = L.decode_table(fm)
    assert sorted(inv) == list(range(npts))
    for o, (lane, j) in inv.items():
        assert L.offset(fm, lane, j) == o


def test_32x32_fragment_index_is_split():
    """j of the 32x32 map occupies two non-adjacent digits: j 0->1 is one row,
    j 3->4 jumps eight rows (the same phenomenon as the worked example)."""
    fm = L.MFMA_32X32X16
    for lane in range(64):
        r0, c0 = fm.coords(lane, 0)
        assert fm.coords(lane, 1) == (r0 + 1, c0)
        assert fm.coords(lane, 4) == (r0 + 8, c0)


def mutant(fm, coords, name="mutant"):
    return L.FragmentMap(name, fm.lanes, fm.per_lane, fm.rows, fm.cols, coords)


def test_enumerator_catches_overlap_and_gap():
    fm = L.M16N8K16
    dropped_j_low = mutant(fm, lambda l, j: (l // 4 + 8 * (j >> 1), 2 * (l % 4)))
    dropped_j_high = mutant(fm, lambda l, j: (l // 4, 2 * (l % 4) + (j & 1)))
    wrong_stride = mutant(fm, lambda l, j: (l // 4 + 4 * (j >> 1), 2 * (l % 4) + (j & 1)))
    for m in (dropped_j_low, dropped_j_high, wrong_stride):
        assert not L.is_bijection(m)
        with pytest.raises(ValueError):
            L.decode_table(m)


def test_enumerator_catches_out_of_tile():
    fm = L.M16N8K16
    transposed = mutant(fm, lambda l, j: (2 * (l % 4) + (j & 1), l // 4 + 8 * (j >> 1)))
    assert not L.is_bijection(transposed)


def test_bijective_but_wrong_map_disagrees_with_numeral():
    """A half-swapped map (j's two bits exchanged) is still a bijection; the page's
    numeral is what catches it."""
    fm = L.M16N8K16
    half_swapped = mutant(fm, lambda l, j: (l // 4 + 8 * (j & 1), 2 * (l % 4) + (j >> 1)))
    assert L.is_bijection(half_swapped)
    bad = sum(L.numeral_value(L.M16N8K16_DIGITS, L.m16n8k16_digit_values(l, j)) != L.offset(half_swapped, l, j)
              for l in range(32) for j in range(4))
    assert bad > 0


@pytest.mark.parametrize("name", ["m16n8k16", "mfma_16x16x32", "mfma_32x32x16"])
def test_strided_placement_disjoint(name):
    """Tiles placed at distinct tile-aligned origins of a row-major matrix with a
    padded leading dimension never share an element."""
    fm = L.MAPS[name]
    ld = 3 * fm.cols + 5
    seen = set()
    for tr in range(3):
        for tc in range(3):
            for lane in range(fm.lanes):
                for j in range(fm.per_lane):
                    o = L.matrix_offset(fm, lane, j, tr * fm.rows, tc * fm.cols, ld)
                    assert o is not None and o not in seen
                    seen.add(o)
    assert len(seen) == 9 * fm.rows * fm.cols


def test_matrix_offset_overflow():
    fm = L.MFMA_16X16X32
    assert L.matrix_offset(fm, 0, 0, 0, 0, 16) == 0
    assert L.matrix_offset(fm, 63, 3, 0, 0, 16) == 15 * 16 + 15
    # column spills past the leading dimension
    assert L.matrix_offset(fm, 15, 0, 0, 8, 16) is None
    # signed 64-bit overflow
    assert L.matrix_offset(fm, 63, 3, (1 << 62), 0, 4) is None
    big = L.matrix_offset(fm, 0, 0, (1 << 62) // 4096 - 1, 0, 4096)
    assert big is not None and big < (1 << 63)
    with pytest.raises(ValueError):
        L.matrix_offset(fm, 0, 0, -1, 0, 16)


# ---- operand fragments (the maps the device probe pins on hardware)

@pytest.mark.parametrize("key", sorted(L.OPERAND_MAPS))
def test_operand_maps_are_bijections_with_inverse(key):
    om = L.OPERAND_MAPS[key]
    assert L.operand_is_bijection(om)
    inv = L.operand_decode_table(om)
    assert sorted(inv) == list(range(om.rows * om.cols))
    for o, (lane, i) in inv.items():
        assert L.operand_offset(om, lane, i) == o


@pytest.mark.parametrize("shape", [0, 1])
def test_operand_maps_are_transposes_of_each_other(shape):
    """A and B of one instruction use the same lane assignment with row and column
    exchanged: lane l supplies A[m][k] and B[k][m] for the same (m, k)."""
    a, b = L.OPERAND_MAPS[(shape, "A")], L.OPERAND_MAPS[(shape, "B")]
    for lane in range(64):
        for i in range(8):
            r, c = a.coords(lane, i)
            assert b.coords(lane, i) == (c, r)
            assert L.operand_offset(a, lane, i) == L.operand_offset(b, lane, i)


@pytest.mark.parametrize("shape,mn,k", [(0, 16, 32), (1, 32, 16)])
def test_operand_maps_cover_k_with_eight_consecutive_elements(shape, mn, k):
    """Each lane's 8 elements are one row (A) of 8 consecutive K positions starting
    at a multiple of 8: the 16-byte register group the MFMA reads."""
    om = L.OPERAND_MAPS[(shape, "A")]
    for lane in range(64):
        pts = [om.coords(lane, i) for i in range(8)]
        assert len({r for r, _ in pts}) == 1
        ks = [c for _, c in pts]
        assert ks == list(range(ks[0], ks[0] + 8)) and ks[0] % 8 == 0 and ks[-1] < k


def test_operand_enumerator_catches_mutants():
    om = L.OPERAND_MAPS[(0, "A")]

    def mut(coords):
        return L.OperandMap("mutant", "A", 64, 8, 16, 32, coords)

    assert not L.operand_is_bijection(mut(lambda l, i: (l % 16, 8 * (l // 16) + (i & 6))))     # dropped i bit
    assert not L.operand_is_bijection(mut(lambda l, i: (l % 16, 4 * (l // 16) + i)))           # wrong K stride
    assert not L.operand_is_bijection(mut(lambda l, i: (8 * (l // 16) + i, l % 16)))           # transposed
    swapped = mut(lambda l, i: (4 * (l % 4) + l // 16, 8 * ((l // 4) % 4) + i))                # lane digits swapped
    assert L.operand_is_bijection(swapped)
    assert any(swapped.coords(l, 0) != om.coords(l, 0) for l in range(64))


@pytest.mark.parametrize("key", sorted(L.OPERAND_MAPS))
def test_operand_matrix_offset_places_the_tile_block(key):
    """Scatter every (lane, i) of one operand fragment through
    operand_matrix_offset into flat storage and read it back with numpy's own
    row-major indexing: the fragment fills exactly the rows x cols block at the
    origin, each element once, and the column-major placement is the transpose
    of the same storage (numpy's .T), holding the same block."""
    om = L.OPERAND_MAPS[key]
    row0, col0, ld = 5, 3, om.cols + om.rows + 11
    rows_total = row0 + om.rows + 2
    cols_total = col0 + om.cols + 2
    ids = {}
    flat_r = np.full(rows_total * ld, -1, dtype=np.int64)        # row-major: (rows_total, ld)
    flat_c = np.full(cols_total * ld, -1, dtype=np.int64)        # column-major: (cols_total, ld)
    for lane in range(om.lanes):
        for i in range(om.per_lane):
            ident = lane * om.per_lane + i
            ids[ident] = True
            o_r = L.operand_matrix_offset(om, lane, i, row0, col0, ld, 0)
            o_c = L.operand_matrix_offset(om, lane, i, row0, col0, ld, 1)
            assert flat_r[o_r] == -1 and flat_c[o_c] == -1
            flat_r[o_r] = ident
            flat_c[o_c] = ident
    mat_r = flat_r.reshape(rows_total, ld)
    mat_c = flat_c.reshape(cols_total, ld).T                      # (ld, cols_total), row index first
    block = (slice(row0, row0 + om.rows), slice(col0, col0 + om.cols))
    assert sorted(mat_r[block].ravel().tolist()) == sorted(ids)
    assert (mat_r >= 0).sum() == om.rows * om.cols               # nothing outside the block
    assert np.array_equal(mat_c[block], mat_r[block])
    assert (mat_c >= 0).sum() == om.rows * om.cols


def test_operand_matrix_offset_orders_and_overflow():
    om = L.OPERAND_MAPS[(1, "B")]       # 16 x 32 (K x N)
    r, c = om.coords(37, 5)
    assert L.operand_matrix_offset(om, 37, 5, 3, 7, 100, 0) == (3 + r) * 100 + 7 + c
    assert L.operand_matrix_offset(om, 37, 5, 3, 7, 100, 1) == (7 + c) * 100 + 3 + r
    assert L.operand_matrix_offset(om, 63, 7, 0, 0, 32, 0) is not None
    assert L.operand_matrix_offset(om, 63, 7, 0, 1, 32, 0) is None            # column spills past ld
    assert L.operand_matrix_offset(om, 63, 7, 17, 0, 32, 1) is None           # row spills past ld (col-major)
    assert L.operand_matrix_offset(om, 0, 0, 1 << 62, 0, 4, 0) is None        # int64 overflow
    with pytest.raises(ValueError):
        L.operand_matrix_offset(om, 0, 0, 0, 0, 16, 2)
