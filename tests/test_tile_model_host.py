"""Host models of the fast GEMM path's tile order, operand extents and epilogue.

These run on the CPU and check the design's index arithmetic for the
configurations the fast paths launch (dense GEMM: 256 x 256 tiles with 4 x 4
waves, 192 x 192 with 3 x 4, 128 x 128, 64 x 64 and 32 x 32 with 2 x 2; split GEMM planes kernel:
128 x 128 with 4 x 4) at tile-multiple and ragged sizes:

  * the XCD-aware tile order (``tile_of`` in csrc/common.hpp) visits every
    tile of the grid exactly once;
  * the direct-to-LDS loads never reach past an operand's minimum storage: the
    buffer extent of a tile panel ends at the last valid element (K-contiguous:
    K elements into row ``valid - 1``; k-major: ``valid`` elements into the last
    K row), and the hardware returns zeros for every dword at or past it;
  * the epilogue (``store_acc_rsrc``) stores every element of the M x N block of
    C exactly once and nothing outside it.  A store's offset is the lane part
    ``(row(lane, 0), col(lane, 0))`` plus the register part ``row(0, v)``; that
    split is checked here against the library's own ``acc_coords``, and the
    rows past the tile's valid rows fall outside the C buffer's extent while
    columns past N are skipped by the per-lane predicate.
"""
import itertools

import pytest

import mma_fragment_layouts_amd as mfl

# (BM, BN, WGM, WGN): the dense fast path's launches and the split planes kernel's
CONFIGS = [(256, 256, 4, 4), (192, 192, 3, 4), (128, 128, 2, 2), (64, 64, 2, 2), (32, 32, 2, 2), (128, 128, 4, 4)]
RAGGED = [(4096, 4096), (4000, 4000), (1000, 520), (300, 1000), (257, 129), (64, 64), (1, 1)]


def tile_of(bid, nwg, tiles_m, tiles_n, group_m=4):
    """Same arithmetic as the device function: renumber so that an XCD's
    workgroups are consecutive, then walk groups of `group_m` tile rows."""
    if nwg % 8 == 0:
        bid = (bid & 7) * (nwg >> 3) + (bid >> 3)
    per_group = group_m * tiles_n
    g = bid // per_group
    first_m = g * group_m
    gsize = min(tiles_m - first_m, group_m)
    in_g = bid - g * per_group
    return first_m + in_g % gsize, in_g // gsize


@pytest.mark.parametrize("tiles_m,tiles_n", [(t, u) for t in (1, 2, 3, 4, 5, 7, 8, 12, 16, 17, 24, 32)
                                             for u in (1, 3, 4, 8, 15, 16, 32)])
def test_tile_order_visits_every_tile_once(tiles_m, tiles_n):
    nwg = tiles_m * tiles_n
    seen = [tile_of(b, nwg, tiles_m, tiles_n) for b in range(nwg)]
    assert sorted(seen) == [(i, j) for i in range(tiles_m) for j in range(tiles_n)]


def test_tile_order_groups_an_xcds_workgroups():
    """At 4096^3 (16 x 16 tiles of 256) the 32 workgroups one XCD receives
    (ids congruent mod 8) cover 4 tile rows x 8 tile columns: 4 A panels and
    8 B panels per XCD L2."""
    for x in range(8):
        tiles = [tile_of(b, 256, 16, 16) for b in range(x, 256, 8)]
        assert len({t[0] for t in tiles}) == 4 and len({t[1] for t in tiles}) == 8


@pytest.mark.parametrize("m,n", RAGGED)
@pytest.mark.parametrize("k", [4096, 4056, 8])
def test_operand_extents_stay_inside_minimum_storage(m, n, k):
    for bm, bn, _, _ in CONFIGS:
        for rows, r_tile in ((m, bm), (n, bn)):
            ld_k = k + (-k) % 8 + 64     # K-contiguous storage: rows x ld, ld >= K
            ld_r = rows + (-rows) % 8    # k-major storage: K x ld, ld >= rows
            for r0 in range(0, rows, r_tile):
                valid = min(rows - r0, r_tile)
                # K-contiguous: base r0*ld, extent (valid-1)*ld + K elements
                end = r0 * ld_k + (valid - 1) * ld_k + k
                assert end <= (rows - 1) * ld_k + k
                # k-major: base r0, extent (K-1)*ld + valid elements
                end = r0 + (k - 1) * ld_r + valid
                assert end <= (k - 1) * ld_r + rows
                # a full panel's extent is what the tile-multiple variant uses
                if valid == r_tile and k % 64 == 0:
                    assert r0 * ld_k + r_tile * ld_k <= rows * ld_k


@pytest.mark.parametrize("shape", [0, 1])
def test_accumulator_offset_splits_into_lane_and_register_parts(shape):
    _, j_count, mn, _ = mfl.mfl_acc_info(shape)   # lanes, J, tile rows, tile columns
    for lane, v in itertools.product(range(64), range(j_count)):
        r, c = mfl.acc_coords(shape, lane, v)
        assert r == mfl.acc_coords(shape, lane, 0)[0] + mfl.acc_coords(shape, 0, v)[0]
        assert c == mfl.acc_coords(shape, lane, 0)[1]


def stored_elements(m, n, ldc, bm, bn, wgm, wgn, shape):
    """Every C element the epilogue writes, per the store offsets and the two clips."""
    _, j_count, mn, _ = mfl.mfl_acc_info(shape)   # lanes, J, tile rows, tile columns
    lane_part = [mfl.acc_coords(shape, lane, 0) for lane in range(64)]
    reg_row = [mfl.acc_coords(shape, 0, v)[0] for v in range(j_count)]
    wm, wn = bm // wgm, bn // wgn
    tm_count, tn_count = (m + bm - 1) // bm, (n + bn - 1) // bn
    out = []
    for tm, tn in itertools.product(range(tm_count), range(tn_count)):
        row0, col0 = tm * bm, tn * bn
        for wave in range(wgm * wgn):
            wr0, wc0 = (wave // wgn) * wm, (wave % wgn) * wn
            wrows = max(0, min(wm, m - (row0 + wr0)))    # C buffer extent: wrows rows of ldc
            ncols = n - (col0 + wc0)                     # per-lane column predicate
            for lane, (lr, lc) in enumerate(lane_part):
                for i in range(wm // mn):
                    for v in range(j_count):
                        r = i * mn + lr + reg_row[v]
                        for j in range(wn // mn):
                            c = lc + j * mn
                            if c >= ncols:
                                continue
                            if r * ldc + c >= wrows * ldc:   # byte offset past the extent: dropped
                                continue
                            out.append((row0 + wr0 + r, col0 + wc0 + c))
    return out


@pytest.mark.parametrize("m,n", [(4000, 520), (257, 129), (300, 1000), (64, 64), (1, 1), (512, 512), (500, 700)])
@pytest.mark.parametrize("shape", [0, 1])
def test_epilogue_stores_each_element_once(m, n, shape):
    ldc = n + 3
    mn = mfl.mfl_acc_info(shape)[2]
    for bm, bn, wgm, wgn in CONFIGS:
        if (bm // wgm) % mn or (bn // wgn) % mn:
            continue   # 48- and 16-wide wave tiles: 16x16x32 only, as the dispatcher launches them
        s = stored_elements(m, n, ldc, bm, bn, wgm, wgn, shape)
        assert len(s) == m * n, (bm, bn)
        assert len(set(s)) == m * n
        assert all(0 <= r < m and 0 <= c < n for r, c in s)
