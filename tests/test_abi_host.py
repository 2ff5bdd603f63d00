"""Host-side tests of libmfl.so: it loads, exports every entry point the header
declares, its layout functions agree bit for bit with the oracle's brute-force
enumeration, and invalid arguments are rejected before any HIP call (so these
run without a GPU)."""
import os
import re

import pytest

from oracle import layouts as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mfl.h")
SHAPES = {0: OL.MFMA_16X16X32, 1: OL.MFMA_32X32X16}


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^MFL_API\s+(?:const\s+char\s*\*|int)\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_and_library_exports_every_entry_point(lib):
    declared = header_functions()
    assert len(declared) >= 15
    so = lib.load()
    for name in declared:
        assert hasattr(so, name), f"{name} declared in mfl.h but not exported"
    assert sorted(lib.EXPORTS) == declared


def test_library_resolves_every_symbol():
    """Binding every symbol at load time catches a kernel whose launch stub was
    never emitted (lazy binding would only fail at the first call)."""
    import ctypes
    from mma_fragment_layouts_amd import _binding
    ctypes.CDLL(_binding.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_version_and_status_strings(lib):
    assert lib.mfl_version() >= 100
    assert lib.status_string(0) == "MFL_OK"
    for st in (-1, -2, -3, -4, -5):
        assert lib.status_string(st).startswith("MFL_E")
    assert "unknown" in lib.status_string(17)


@pytest.mark.parametrize("shape", [0, 1])
def test_acc_info(lib, shape):
    fm = SHAPES[shape]
    assert lib.mfl_acc_info(shape) == (fm.lanes, fm.per_lane, fm.rows, fm.cols)


@pytest.mark.parametrize("shape", [0, 1])
def test_coords_offsets_decode_match_oracle_exhaustively(lib, shape):
    """Every (lane, j): the library's numeral-form coordinates and offsets equal
    the oracle's row/col enumeration; decode equals the oracle's inverted table."""
    fm = SHAPES[shape]
    inv = OL.decode_table(fm)
    for lane in range(fm.lanes):
        for j in range(fm.per_lane):
            assert lib.acc_coords(shape, lane, j) == fm.coords(lane, j)
            assert lib.acc_offset(shape, lane, j) == OL.offset(fm, lane, j)
    for o in range(fm.rows * fm.cols):
        assert lib.acc_decode(shape, o) == inv[o]


@pytest.mark.parametrize("shape", [0, 1])
def test_six_layout_properties(lib, shape):
    """The six checks of the cuda-oxide page's "Tests" section, on the library."""
    fm = SHAPES[shape]
    L, J, R, Cc = lib.mfl_acc_info(shape)
    pts = [(l, j) for l in range(L) for j in range(J)]
    # 1. bijection via an ownership map (no overlap, no gap)
    own = [[0] * Cc for _ in range(R)]
    for l, j in pts:
        r, c = lib.acc_coords(shape, l, j)
        own[r][c] += 1
    assert all(v == 1 for row in own for v in row)
    # 2. numeral form agrees with the row/col form
    for l, j in pts:
        r, c = lib.acc_coords(shape, l, j)
        assert lib.acc_offset(shape, l, j) == r * Cc + c
    # 3. decode is a true inverse on all points (both directions)
    for l, j in pts:
        assert lib.acc_decode(shape, lib.acc_offset(shape, l, j)) == (l, j)
    for o in range(R * Cc):
        assert lib.acc_offset(shape, *lib.acc_decode(shape, o)) == o
    # 4. the fragment index is split: j 0->1 moves one row; the next digit of j
    #    (j 0->J/... ) moves further, in rows, never in columns
    for l in range(L):
        r0, c0 = lib.acc_coords(shape, l, 0)
        assert lib.acc_coords(shape, l, 1) == (r0 + 1, c0)
        if shape == 1:
            assert lib.acc_coords(shape, l, 4) == (r0 + 8, c0)
    # 5. disjointness preserved under strided placement
    ld = 3 * Cc + 8
    seen = set()
    for tr in range(3):
        for tc in range(3):
            for l, j in pts:
                o = lib.acc_matrix_offset(shape, l, j, tr * R, tc * Cc, ld)
                assert o is not None and o not in seen
                assert o == OL.matrix_offset(fm, l, j, tr * R, tc * Cc, ld)
                seen.add(o)
    # 6. overflow rejection
    assert lib.acc_matrix_offset(shape, L - 1, J - 1, 0, Cc, 2 * Cc - 1) is None   # spills past ld
    assert lib.acc_matrix_offset(shape, L - 1, J - 1, 1 << 62, 0, 4) is None        # int64 overflow
    assert OL.matrix_offset(fm, L - 1, J - 1, 1 << 62, 0, 4) is None


def test_matrix_offset_matches_oracle_on_random_origins(lib):
    import random
    rnd = random.Random(5)
    for _ in range(2000):
        shape = rnd.randint(0, 1)
        fm = SHAPES[shape]
        lane, j = rnd.randrange(64), rnd.randrange(fm.per_lane)
        ld = rnd.choice([fm.cols, fm.cols + 1, 4096, 4160, (1 << 40) + 7])
        row0 = rnd.choice([0, 1, 17, 4095, (1 << 22), (1 << 62) // ld])
        col0 = rnd.choice([0, 1, ld - fm.cols, max(0, ld - 1)])
        assert lib.acc_matrix_offset(shape, lane, j, row0, col0, ld) == OL.matrix_offset(fm, lane, j, row0, col0, ld)


def test_layout_argument_errors(lib):
    for bad in [(2, 0, 0), (-1, 0, 0), (0, 64, 0), (0, -1, 0), (0, 0, 4), (1, 0, 16)]:
        with pytest.raises(lib.MflError) as e:
            lib.acc_coords(*bad)
        assert e.value.status == lib.EINVAL
    with pytest.raises(lib.MflError):
        lib.acc_decode(0, 256)
    with pytest.raises(lib.MflError):
        lib.acc_decode(1, -1)
    with pytest.raises(lib.MflError):
        lib.acc_matrix_offset(0, 0, 0, -1, 0, 16)
    with pytest.raises(lib.MflError):
        lib.acc_matrix_offset(0, 0, 0, 0, 0, 0)


OPS = {0: "A", 1: "B"}


@pytest.mark.parametrize("operand", [0, 1])
@pytest.mark.parametrize("shape", [0, 1])
def test_operand_info(lib, shape, operand):
    om = OL.OPERAND_MAPS[(shape, OPS[operand])]
    assert lib.mfl_operand_info(shape, operand) == (om.lanes, om.per_lane, om.rows, om.cols)


@pytest.mark.parametrize("operand", [0, 1])
@pytest.mark.parametrize("shape", [0, 1])
def test_operand_coords_offsets_decode_match_oracle_exhaustively(lib, shape, operand):
    om = OL.OPERAND_MAPS[(shape, OPS[operand])]
    inv = OL.operand_decode_table(om)
    for lane in range(64):
        for i in range(8):
            assert lib.operand_coords(shape, operand, lane, i) == om.coords(lane, i)
            assert lib.operand_offset(shape, operand, lane, i) == OL.operand_offset(om, lane, i)
    for o in range(om.rows * om.cols):
        assert lib.operand_decode(shape, operand, o) == inv[o]


@pytest.mark.parametrize("operand", [0, 1])
@pytest.mark.parametrize("shape", [0, 1])
def test_six_operand_layout_properties(lib, shape, operand):
    """The cuda-oxide page's six checks ("Tests" section), on the operand maps."""
    om = OL.OPERAND_MAPS[(shape, OPS[operand])]
    L, E, R, Cc = lib.mfl_operand_info(shape, operand)
    kdim = Cc if operand == 0 else R
    pts = [(l, i) for l in range(L) for i in range(E)]
    # 1. bijection via an ownership map
    own = [[0] * Cc for _ in range(R)]
    for l, i in pts:
        r, c = lib.operand_coords(shape, operand, l, i)
        own[r][c] += 1
    assert all(v == 1 for row in own for v in row)
    # 2. numeral form agrees with the row/col form (K-contiguous storage)
    for l, i in pts:
        r, c = lib.operand_coords(shape, operand, l, i)
        mn, k = (r, c) if operand == 0 else (c, r)
        assert lib.operand_offset(shape, operand, l, i) == mn * kdim + k
    # 3. decode is a true inverse on all points, both directions
    for l, i in pts:
        assert lib.operand_decode(shape, operand, lib.operand_offset(shape, operand, l, i)) == (l, i)
    for o in range(R * Cc):
        assert lib.operand_offset(shape, operand, *lib.operand_decode(shape, operand, o)) == o
    # 4. the element index moves along K only; the lane's high digit moves K by 8
    mnn = 64 * 8 // kdim
    for l in range(L):
        r0, c0 = lib.operand_coords(shape, operand, l, 0)
        step = (0, 1) if operand == 0 else (1, 0)
        assert lib.operand_coords(shape, operand, l, 1) == (r0 + step[0], c0 + step[1])
        if l + mnn < L:
            r1, c1 = lib.operand_coords(shape, operand, l + mnn, 0)
            assert (r1 - r0, c1 - c0) == (8 * step[0], 8 * step[1])
    # 5. disjointness under strided placement, both orders
    for order in (0, 1):
        ld = 3 * (Cc if order == 0 else R) + 8
        seen = set()
        for tr in range(3):
            for tc in range(3):
                for l, i in pts:
                    o = lib.operand_matrix_offset(shape, operand, l, i, tr * R, tc * Cc, ld, order)
                    assert o is not None and o not in seen
                    assert o == OL.operand_matrix_offset(om, l, i, tr * R, tc * Cc, ld, order)
                    seen.add(o)
    # 6. overflow rejection
    assert lib.operand_matrix_offset(shape, operand, L - 1, E - 1, 0, Cc, 2 * Cc - 1, 0) is None
    assert lib.operand_matrix_offset(shape, operand, L - 1, E - 1, R, 0, 2 * R - 1, 1) is None
    assert lib.operand_matrix_offset(shape, operand, L - 1, E - 1, 1 << 62, 0, 64, 0) is None


def test_operand_matrix_offset_matches_oracle_on_random_origins(lib):
    import random
    rnd = random.Random(7)
    for _ in range(2000):
        shape, operand, order = rnd.randint(0, 1), rnd.randint(0, 1), rnd.randint(0, 1)
        om = OL.OPERAND_MAPS[(shape, OPS[operand])]
        lane, i = rnd.randrange(64), rnd.randrange(8)
        inner = om.cols if order == 0 else om.rows
        ld = rnd.choice([inner, inner + 1, 4096, 4160, (1 << 40) + 7])
        o_outer = rnd.choice([0, 1, 17, 4095, (1 << 22), (1 << 62) // ld])
        o_inner = rnd.choice([0, 1, ld - inner, max(0, ld - 1)])
        row0, col0 = (o_outer, o_inner) if order == 0 else (o_inner, o_outer)
        assert (lib.operand_matrix_offset(shape, operand, lane, i, row0, col0, ld, order)
                == OL.operand_matrix_offset(om, lane, i, row0, col0, ld, order))


def test_operand_argument_errors(lib):
    for bad in [(2, 0, 0, 0), (0, 2, 0, 0), (0, -1, 0, 0), (0, 0, 64, 0), (1, 1, 0, 8), (1, 0, 0, -1)]:
        with pytest.raises(lib.MflError) as e:
            lib.operand_coords(*bad)
        assert e.value.status == lib.EINVAL
    with pytest.raises(lib.MflError):
        lib.operand_decode(0, 0, 512)
    with pytest.raises(lib.MflError):
        lib.operand_decode(1, 1, -1)
    with pytest.raises(lib.MflError):
        lib.operand_matrix_offset(0, 0, 0, 0, 0, 0, 16, 2)
    with pytest.raises(lib.MflError):
        lib.operand_matrix_offset(0, 1, 0, 0, -1, 0, 16, 0)


FAKE = 1 << 20  # a 16-byte aligned non-null value; never dereferenced (rejected first)


@pytest.mark.parametrize("call,status", [
    # bad dtype / shape / orders / accumulate flag
    (lambda m: m.gemm_tile_mma(7, 64, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma_shape(2, 1, 64, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 64, 3, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64, accumulate=2), -1),
    # null operands, misaligned pointer, ld too small, ld not a multiple of 8, negative sizes
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, 0, 64, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE + 2, 64, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 56, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 68, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 32), -1),
    (lambda m: m.gemm_tile_mma(1, -1, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 64, 64, 64, FAKE, 64, 0, FAKE, 64, 1, 0, 64), -1),
    (lambda m: m.gemm_tile_mma(1, 1 << 31, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64), -3),
    # block repeat: unsupported tile, non-multiple output
    (lambda m: m.gemm_block_repeat(0, 48, 48, 64, 128, 64, 2048, 2048, FAKE, FAKE, FAKE), -3),
    (lambda m: m.gemm_block_repeat(0, 64, 64, 64, 96, 64, 2048, 2048, FAKE, FAKE, FAKE), -3),
    (lambda m: m.gemm_block_repeat(0, 64, 64, 64, 128, 64, 2000, 2048, FAKE, FAKE, FAKE), -3),
    (lambda m: m.gemm_block_repeat(0, 64, 64, 64, 128, -1, 2048, 2048, FAKE, FAKE, FAKE), -1),
    (lambda m: m.gemm_block_repeat_lds_api(0, 48, 48, 64, 128, 64, 2048, 2048, FAKE, FAKE, FAKE), -3),
    (lambda m: m.gemm_block_repeat_lds_api(2, 64, 64, 64, 128, 64, 2048, 2048, FAKE, FAKE, FAKE), -1),
    (lambda m: m.gemm_block_repeat_lds_api(0, 64, 64, 64, 128, 64, 2048, 2048, FAKE + 2, FAKE, FAKE), -1),
    # split: chains beyond the products, lo*lo without two split operands, bad mode, ld % 4
    (lambda m: m.gemm_split_fp32(1, 64, 64, 64, FAKE, 64, 0, 1, FAKE, 64, 1, 0, 3, 0, FAKE, 64), -1),
    (lambda m: m.gemm_split_fp32(1, 64, 64, 64, FAKE, 64, 0, 1, FAKE, 64, 1, 0, 1, 1, FAKE, 64), -1),
    (lambda m: m.gemm_split_fp32(1, 64, 64, 64, FAKE, 64, 0, 2, FAKE, 64, 1, 0, 1, 0, FAKE, 64), -1),
    (lambda m: m.gemm_split_fp32(1, 64, 64, 64, FAKE, 66, 0, 1, FAKE, 64, 1, 1, 3, 0, FAKE, 64), -1),
    (lambda m: m.gemm_split_fp32(1, 64, 64, 64, FAKE, 64, 0, 1, FAKE, 64, 1, 1, 0, 0, FAKE, 64), -1),
    # attention: unsupported sizes, bad chains, small workspace, misaligned workspace
    (lambda m: m.attention_split_fp32(2048, 32768, 64, FAKE, FAKE, FAKE, 2, 1, FAKE, FAKE, 1 << 40), -3),
    (lambda m: m.attention_split_fp32(2000, 32768, 128, FAKE, FAKE, FAKE, 2, 0, FAKE, FAKE, 1 << 40), -3),
    (lambda m: m.attention_split_fp32(2048, 32768, 128, FAKE, FAKE, FAKE, 3, 1, FAKE, FAKE, 1 << 40), -1),
    (lambda m: m.attention_split_fp32(2048, 32768, 128, FAKE, FAKE, FAKE, 2, 3, FAKE, FAKE, 1 << 40), -1),
    (lambda m: m.attention_split_fp32(128, 1 << 24, 128, FAKE, FAKE, FAKE, 2, 1, FAKE, FAKE, 1 << 40), -3),
    (lambda m: m.attention_split_fp32(2048, 32768, 128, FAKE, FAKE, FAKE, 2, 0, FAKE, FAKE, 1024), -1),
    (lambda m: m.attention_split_fp32(2048, 32768, 128, FAKE, FAKE, FAKE, 2, 1, FAKE, FAKE, 1024), -1),
    (lambda m: m.attention_split_fp32(2048, 32768, 128, FAKE, FAKE, FAKE, 2, 1, FAKE, FAKE + 16, 1 << 40), -1),
    # quantise / split: misaligned, negative n, bad dtype
    (lambda m: m.quantize_fp32(1, FAKE + 4, FAKE, 16), -1),
    (lambda m: m.quantize_fp32(1, FAKE, FAKE, -1), -1),
    (lambda m: m.split_fp32(3, FAKE, FAKE, FAKE, 16), -1),
    # strided store: spill past ldc, probe: bad shape
    (lambda m: m.acc_store_strided(0, FAKE, FAKE, 0, 8, 16), -2),
    (lambda m: m.acc_store_strided(1, FAKE, FAKE, (1 << 62), 0, 64), -2),
    (lambda m: m.mfma_probe(2, 0, FAKE, FAKE, None, FAKE), -1),
    # strided operand load: contiguous extent past ld (both orders), int64 overflow, bad operand/order, odd pointer
    (lambda m: m.operand_load_strided(0, 0, FAKE, 0, 1, 32, 0, FAKE), -2),
    (lambda m: m.operand_load_strided(0, 1, FAKE, 1, 0, 32, 1, FAKE), -2),
    (lambda m: m.operand_load_strided(1, 0, FAKE, 1 << 62, 0, 64, 0, FAKE), -2),
    (lambda m: m.operand_load_strided(0, 2, FAKE, 0, 0, 64, 0, FAKE), -1),
    (lambda m: m.operand_load_strided(0, 0, FAKE, 0, 0, 64, 2, FAKE), -1),
    (lambda m: m.operand_load_strided(0, 0, FAKE + 1, 0, 0, 64, 0, FAKE), -1),
    (lambda m: m.operand_load_strided(0, 0, FAKE, -1, 0, 64, 0, FAKE), -1),
])
def test_device_entry_points_reject_bad_arguments(lib, call, status):
    with pytest.raises(lib.MflError) as e:
        call(lib)
    assert e.value.status == status


def test_empty_problems_are_noops_without_a_device(lib):
    # M = 0 or N = 0: nothing to do, no HIP call
    lib.gemm_tile_mma(1, 0, 64, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64)
    lib.gemm_tile_mma(1, 64, 0, 64, FAKE, 64, 0, FAKE, 64, 1, FAKE, 64)
    lib.gemm_split_fp32(1, 0, 64, 64, FAKE, 64, 0, 1, FAKE, 64, 1, 1, 3, 0, FAKE, 64)
    lib.gemm_block_repeat(0, 64, 64, 64, 128, 64, 0, 0, FAKE, FAKE, FAKE)
    lib.quantize_fp32(1, FAKE, FAKE, 0)


def test_split_planes_workspace_size(lib):
    R_, C_, S_, Rd = lib.ROW_MAJOR, lib.COL_MAJOR, lib.SPLIT, lib.ROUND
    al = lambda x: (x + 255) // 256 * 256
    # applicable: four 16-bit planes in the operands' storage shapes (A: m rows
    # row-major, k rows column-major; B: n rows column-major, k rows row-major)
    # of ld elements each, 256-aligned
    assert lib.gemm_split_fp32_workspace_bytes(512, 384, 640, 648, R_, S_, 664, C_, S_, 384) == \
        2 * al(512 * 648 * 2) + 2 * al(384 * 664 * 2)
    assert lib.gemm_split_fp32_workspace_bytes(512, 384, 640, 520, C_, S_, 392, R_, S_, 384) == \
        2 * al(640 * 520 * 2) + 2 * al(640 * 392 * 2)
    assert lib.gemm_split_fp32_workspace_bytes(512, 384, 640, 648, R_, S_, 392, R_, S_, 384) == \
        2 * al(512 * 648 * 2) + 2 * al(640 * 392 * 2)
    # ragged M, N and K (a multiple of 8) take the planes path as well
    assert lib.gemm_split_fp32_workspace_bytes(500, 390, 600, 648, R_, S_, 664, C_, S_, 392) == \
        2 * al(500 * 648 * 2) + 2 * al(390 * 664 * 2)
    assert lib.gemm_split_fp32_workspace_bytes(504, 392, 600, 512, C_, S_, 400, R_, S_, 392) == \
        2 * al(600 * 512 * 2) + 2 * al(600 * 400 * 2)
    # not applicable: no workspace (the split-on-load kernel runs)
    for args in [(512, 384, 640, 648, R_, Rd, 664, C_, S_, 384),   # A rounded
                 (512, 384, 602, 648, R_, S_, 664, C_, S_, 384),   # K % 8
                 (500, 384, 640, 504, C_, S_, 664, C_, S_, 384),   # column-major A, M % 8
                 (512, 390, 640, 648, R_, S_, 392, R_, S_, 392),   # row-major B, N % 8
                 (512, 384, 640, 644, R_, S_, 664, C_, S_, 384)]:  # lda % 8
        assert lib.gemm_split_fp32_workspace_bytes(*args) == 0
    with pytest.raises(lib.MflError):
        lib.gemm_split_fp32_workspace_bytes(512, 384, 640, 648, 2, S_, 664, C_, S_, 384)
    with pytest.raises(lib.MflError):
        lib.gemm_split_fp32_workspace_bytes(512, 384, 640, 648, R_, 3, 664, C_, S_, 384)


@pytest.mark.parametrize("ws,wsb", [(FAKE, 1024), (0, 1 << 40), (FAKE + 16, 1 << 40)])
def test_split_planes_rejects_bad_workspace(lib, ws, wsb):
    with pytest.raises(lib.MflError) as e:
        lib.gemm_split_fp32_ws(1, 512, 384, 640, FAKE, 648, lib.ROW_MAJOR, lib.SPLIT, FAKE, 664, lib.COL_MAJOR,
                               lib.SPLIT, 3, 0, FAKE, 384, 0, ws, wsb)
    assert e.value.status == lib.EINVAL


def test_attention_workspace_size(lib):
    b = lib.attention_workspace_bytes(2048, 32768, 128, 0)
    assert b >= 2048 * 32768 * 4 + 2 * 2048 * 4 + 2048 * 128 * 4
    f = lib.attention_workspace_bytes(2048, 32768, 128, 1)
    # fp16 K and V plus per-slice partial O, m, l: far below the materialised scores
    assert 2 * 32768 * 128 * 2 < f < b // 4
    with pytest.raises(lib.MflError):
        lib.attention_workspace_bytes(2048, 32768, 96, 1)
    # the fused kernel's 32-bit buffer extent: nk * 128 * 2 bytes must fit
    assert lib.attention_workspace_bytes(128, (1 << 24) - 128, 128, 1) > 0
    for algo in (1, 2):
        with pytest.raises(lib.MflError) as e:
            lib.attention_workspace_bytes(128, 1 << 24, 128, algo)
        assert e.value.status == lib.EUNSUPPORTED
    assert lib.attention_workspace_bytes(128, 1 << 24, 128, 0) > 0
    skv = lib.attention_workspace_bytes(2048, 32768, 128, 2)
    assert skv == f + 2 * 32768 * 128 * 2      # K and V lo planes on top
    with pytest.raises(lib.MflError):
        lib.attention_workspace_bytes(2048, 32768, 128, 5)
    with pytest.raises(lib.MflError):
        lib.attention_workspace_bytes(2048, 32768, 128, 3)


def test_plain_c_program_uses_the_header_and_library(tmp_path):
    """include/mfl.h is valid C99 (pedantic, warnings as errors) and the host
    calls work from a C program linked against libmfl.so (tests/c)."""
    import shutil
    import subprocess
    from mma_fragment_layouts_amd import _binding
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    libdir = os.path.dirname(_binding.LIB_PATH)
    exe = tmp_path / "abi_host_check"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "abi_host_check.c"), "-L", libdir, "-lmfl",
                    f"-Wl,-rpath,{libdir}", "-o", str(exe)], check=True, capture_output=True, text=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, run.stderr
    assert "ok" in run.stdout


def device_program_command(cc, out):
    """Compile line of tests/c/abi_device_gemm.c: plain C99 against mfl.h and
    the HIP runtime's C API, linked with libmfl.so and libamdhip64."""
    from mma_fragment_layouts_amd import _binding
    libdir = os.path.dirname(_binding.LIB_PATH)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(rocm, "include"), os.path.join(ROOT, "tests", "c", "abi_device_gemm.c"), "-L", libdir,
            "-lmfl", "-L", os.path.join(rocm, "lib"), "-lamdhip64", "-lm", f"-Wl,-rpath,{libdir}",
            f"-Wl,-rpath,{os.path.join(rocm, 'lib')}", "-o", str(out)]


def test_plain_c_device_program_builds(tmp_path):
    """The device-side C example (run by the GPU tests) compiles warning-free."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None or not os.path.exists("/opt/rocm/include/hip/hip_runtime_api.h"):
        pytest.skip("no C compiler or HIP headers on this host")
    r = subprocess.run(device_program_command(cc, tmp_path / "abi_device_gemm"), capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_host_tensors_are_refused_before_the_library_is_called(lib):
    """A host (CPU) tensor's address must never reach a kernel: the binding
    raises before calling into the library."""
    import torch
    a = torch.zeros((64, 64), dtype=torch.int16)
    c = torch.zeros((64, 64), dtype=torch.float32)
    with pytest.raises(TypeError, match="host memory"):
        lib.gemm_tile_mma(lib.BF16, 64, 64, 64, a, 64, lib.ROW_MAJOR, a, 64, lib.COL_MAJOR, c, 64, 0, None)
    with pytest.raises(TypeError, match="host memory"):
        lib.quantize_fp32(lib.BF16, c, a, 64, None)


class _DeviceTensorStandIn:
    """Looks like a device tensor to the binding (is_cuda, storage size) but has
    no memory behind it; only used where the binding must refuse the call."""
    is_cuda = True

    def __init__(self, nbytes, elem=2, offset=0):
        self._nbytes, self._elem, self._offset = nbytes, elem, offset

    def untyped_storage(self):
        outer = self

        class _S:
            def nbytes(self):
                return outer._nbytes
        return _S()

    def storage_offset(self):
        return self._offset

    def element_size(self):
        return self._elem

    def data_ptr(self):
        raise AssertionError("the binding must refuse before taking the pointer")


def test_undersized_tensors_are_refused_before_the_library_is_called(lib):
    T = _DeviceTensorStandIn
    m = n = k = 256
    ok16, ok32 = T(m * k * 2), T(m * n * 4, elem=4)
    # C one element short (ldc 256: 256 * 256 fp32 needed)
    with pytest.raises(ValueError, match="`c`"):
        lib.gemm_tile_mma(lib.BF16, m, n, k, ok16, k, lib.ROW_MAJOR, ok16, k, lib.COL_MAJOR,
                          T(m * n * 4 - 4, elem=4), n, 0, None)
    # A stored with a padded leading dimension needs (m - 1) * lda + k elements
    with pytest.raises(ValueError, match="`a`"):
        lib.gemm_tile_mma(lib.BF16, m, n, k, T(m * k * 2), k + 64, lib.ROW_MAJOR, ok16, k, lib.COL_MAJOR, ok32, n, 0,
                          None)
    # a view that starts inside its storage has less room
    with pytest.raises(ValueError, match="`b`"):
        lib.gemm_tile_mma(lib.BF16, m, n, k, ok16, k, lib.ROW_MAJOR, T(m * k * 2, offset=8), k, lib.COL_MAJOR, ok32,
                          n, 0, None)
    with pytest.raises(ValueError, match="`out`"):
        lib.quantize_fp32(lib.BF16, T(1024 * 4, elem=4), T(1023 * 2), 1024, None)
    with pytest.raises(ValueError, match="`workspace`"):
        lib.gemm_split_fp32_ws(lib.BF16, m, n, k, T(m * k * 4, elem=4), k, lib.ROW_MAJOR, lib.SPLIT,
                               T(n * k * 4, elem=4), k, lib.COL_MAJOR, lib.SPLIT, 2, 0, ok32, n, 0, T(100, elem=1), 4096,
                               None)
    with pytest.raises(ValueError, match="`v`"):
        lib.attention_split_fp32(128, 256, 128, T(128 * 128 * 4, elem=4), T(256 * 128 * 4, elem=4),
                                 T(255 * 128 * 4, elem=4), 2, 1, T(128 * 128 * 4, elem=4), T(1 << 20, elem=1), 1 << 20,
                                 None)


def test_extent_of_stored_operands():
    from mma_fragment_layouts_amd import _binding as B
    assert B._op(3, 5, 8, B.ROW_MAJOR, 2) == ((3 - 1) * 8 + 5) * 2
    assert B._op(3, 5, 8, B.COL_MAJOR, 2) == ((5 - 1) * 8 + 3) * 2
    assert B._op(0, 5, 8, B.ROW_MAJOR, 2) == 0
    assert B._extent(4, 4, 4, 4) == 64


def test_undersized_probe_buffers_are_refused(lib):
    T = _DeviceTensorStandIn
    frag = T(64 * 8 * 2)
    with pytest.raises(ValueError, match="`acc`"):   # 32x32x16: 16 fp32 per lane
        lib.mfma_probe(1, lib.F16, frag, frag, None, T(64 * 4 * 4, elem=4), None)
    with pytest.raises(ValueError, match="`frag`"):
        lib.operand_load_strided(0, 0, T(1 << 20), 0, 0, 64, lib.ROW_MAJOR, T(64 * 8 * 2 - 2), None)
    with pytest.raises(ValueError, match="`c`"):     # 16x16 tile at (16, 16) of an ld-32 matrix
        lib.acc_store_strided(0, T(64 * 4 * 4, elem=4), T((31 * 32 + 31) * 4, elem=4), 16, 16, 32, None)
