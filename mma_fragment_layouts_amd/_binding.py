"""ctypes binding of libmfl.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/mfl.h)
and does nothing but convert arguments (device pointers from ints or from
objects with ``data_ptr()``, streams from ints or from objects with
``cuda_stream``), call the library and turn a non-zero status into
``MflError``.  Tensor arguments are also checked, before the call, to be in
device memory and to hold the region the call touches (the C ABI sees plain
pointers and cannot).  All computation happens in the library's HIP kernels; if the
library is missing, the first call raises.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Tuple

# MFL_LIBRARY overrides the library file (the host-sanitizer test loads an
# instrumented build through it); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("MFL_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                         "libmfl.so")

# enums (values fixed by include/mfl.h)
OK, EINVAL, EOVERFLOW, EUNSUPPORTED, EHIP, ESCRATCH = 0, -1, -2, -3, -4, -5
MFMA_16X16X32, MFMA_32X32X16 = 0, 1
F16, BF16 = 0, 1
ROW_MAJOR, COL_MAJOR = 0, 1
ROUND, SPLIT = 0, 1
ATTN_MATERIALISED, ATTN_FUSED, ATTN_FUSED_SPLIT_KV = 0, 1, 2
OPERAND_A, OPERAND_B = 0, 1

_i32, _i64, _vp = C.c_int, C.c_int64, C.c_void_p
_pi32, _pi64 = C.POINTER(C.c_int), C.POINTER(C.c_int64)

_SIGNATURES = {
    "mfl_status_string": (C.c_char_p, [_i32]),
    "mfl_version": (_i32, []),
    "mfl_acc_info": (_i32, [_i32, _pi32, _pi32, _pi32, _pi32]),
    "acc_coords": (_i32, [_i32, _i32, _i32, _pi32, _pi32]),
    "acc_offset": (_i32, [_i32, _i32, _i32, _pi32]),
    "acc_decode": (_i32, [_i32, _i32, _pi32, _pi32]),
    "acc_matrix_offset": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _pi64]),
    "mfl_operand_info": (_i32, [_i32, _i32, _pi32, _pi32, _pi32, _pi32]),
    "operand_coords": (_i32, [_i32, _i32, _i32, _i32, _pi32, _pi32]),
    "operand_offset": (_i32, [_i32, _i32, _i32, _i32, _pi32]),
    "operand_decode": (_i32, [_i32, _i32, _i32, _pi32, _pi32]),
    "operand_matrix_offset": (_i32, [_i32, _i32, _i32, _i32, _i64, _i64, _i64, _i32, _pi64]),
    "operand_load_strided": (_i32, [_i32, _i32, _vp, _i64, _i64, _i64, _i32, _vp, _vp]),
    "acc_store_strided": (_i32, [_i32, _vp, _vp, _i64, _i64, _i64, _vp]),
    "mfma_probe": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "mfma_rate_probe": (_i32, [_i32, _i32, C.c_uint32, _vp, _vp]),
    "quantize_fp32": (_i32, [_i32, _vp, _vp, _i64, _vp]),
    "split_fp32": (_i32, [_i32, _vp, _vp, _vp, _i64, _vp]),
    "gemm_tile_mma": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _vp, _i64, _i32, _vp]),
    "gemm_tile_mma_shape": (_i32, [_i32, _i32, _i64, _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i32, _vp, _i64,
                                   _i32, _vp]),
    "gemm_block_repeat": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp]),
    "gemm_block_repeat_lds_api": (_i32, [_i32, _i32, _i32, _i32, _i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp]),
    "gemm_split_fp32": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _i64, _i32, _i32, _i32, _i32,
                               _vp, _i64, _i32, _vp]),
    "gemm_split_fp32_workspace_bytes": (_i32, [_i64, _i64, _i64, _i64, _i32, _i32, _i64, _i32, _i32, _i64, _pi64]),
    "gemm_split_fp32_ws": (_i32, [_i32, _i64, _i64, _i64, _vp, _i64, _i32, _i32, _vp, _i64, _i32, _i32, _i32, _i32,
                                  _vp, _i64, _i32, _vp, _i64, _vp]),
    "attention_workspace_bytes": (_i32, [_i64, _i64, _i64, _i32, _pi64]),
    "attention_split_fp32": (_i32, [_i64, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i64, _vp]),
    "attention_split_fp32_static": (_i32, [_i64, _i64, _i64, _vp, _vp, _vp, _i32, _i32, _vp, _vp]),
}
EXPORTS = tuple(_SIGNATURES)

_lib: Optional[C.CDLL] = None


class MflError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: {status_string(status)} (status {status})")


def library_path() -> str:
    return LIB_PATH


def load() -> C.CDLL:
    """Load libmfl.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmfl.so not found at {LIB_PATH}; build it with "
                               "`python -m mma_fragment_layouts_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        # a host tensor's address handed to a kernel would fault the GPU
        if getattr(x, "is_cuda", True) is False:
            raise TypeError("expected a device tensor, got one in host memory")
        return x.data_ptr()
    raise TypeError(f"expected a device pointer (int or tensor), got {type(x)}")


def _room(x) -> Optional[int]:
    """Bytes addressable from a tensor's data pointer (to the end of its
    storage), or None when x is a plain integer pointer."""
    if not hasattr(x, "untyped_storage"):
        return None
    return x.untyped_storage().nbytes() - x.storage_offset() * x.element_size()


def _extent(outer: int, inner: int, ld: int, elem: int) -> int:
    """Bytes spanned by `outer` rows of `ld` elements whose last row holds
    `inner` elements (an operand's minimum storage)."""
    return 0 if outer <= 0 or inner <= 0 else ((outer - 1) * ld + inner) * elem


def _op(rows: int, cols: int, ld: int, order: int, elem: int) -> int:
    """Minimum storage of a rows x cols matrix stored in `order`."""
    return _extent(rows, cols, ld, elem) if order == ROW_MAJOR else _extent(cols, rows, ld, elem)


def _need(fn: str, **bufs) -> None:
    """Raise before the call if a tensor argument is smaller than the region the
    call will touch: a kernel would otherwise read or write past it."""
    for name, (x, nbytes) in bufs.items():
        room = _room(x)
        if room is not None and nbytes > room:
            raise ValueError(f"{fn}: `{name}` needs {nbytes} bytes from its data pointer; the tensor holds {room}")


def _layout_info(fn, *args) -> Optional[Tuple[int, int, int, int]]:
    """(lanes, per_lane, rows, cols) from an info call, or None if it fails."""
    v = [C.c_int() for _ in range(4)]
    if fn(*args, *[C.byref(x) for x in v]) != OK:
        return None
    return tuple(x.value for x in v)


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError(f"expected a stream handle, got {type(s)}")


def _check(st: int, fn: str) -> None:
    if st != OK:
        raise MflError(st, fn)


def status_string(status: int) -> str:
    return load().mfl_status_string(status).decode()


def mfl_status_string(status: int) -> str:
    return status_string(status)


def mfl_version() -> int:
    return load().mfl_version()


def mfl_acc_info(shape: int) -> Tuple[int, int, int, int]:
    v = [C.c_int() for _ in range(4)]
    _check(load().mfl_acc_info(shape, *[C.byref(x) for x in v]), "mfl_acc_info")
    return tuple(x.value for x in v)


def acc_coords(shape: int, lane: int, j: int) -> Tuple[int, int]:
    r, c = C.c_int(), C.c_int()
    _check(load().acc_coords(shape, lane, j, C.byref(r), C.byref(c)), "acc_coords")
    return r.value, c.value


def acc_offset(shape: int, lane: int, j: int) -> int:
    o = C.c_int()
    _check(load().acc_offset(shape, lane, j, C.byref(o)), "acc_offset")
    return o.value


def acc_decode(shape: int, offset: int) -> Tuple[int, int]:
    lane, j = C.c_int(), C.c_int()
    _check(load().acc_decode(shape, offset, C.byref(lane), C.byref(j)), "acc_decode")
    return lane.value, j.value


def acc_matrix_offset(shape: int, lane: int, j: int, row0: int, col0: int, ld: int) -> Optional[int]:
    """Strided destination, or None when the library reports MFL_EOVERFLOW."""
    o = C.c_int64()
    st = load().acc_matrix_offset(shape, lane, j, row0, col0, ld, C.byref(o))
    if st == EOVERFLOW:
        return None
    _check(st, "acc_matrix_offset")
    return o.value


def mfl_operand_info(shape: int, operand: int) -> Tuple[int, int, int, int]:
    v = [C.c_int() for _ in range(4)]
    _check(load().mfl_operand_info(shape, operand, *[C.byref(x) for x in v]), "mfl_operand_info")
    return tuple(x.value for x in v)


def operand_coords(shape: int, operand: int, lane: int, i: int) -> Tuple[int, int]:
    r, c = C.c_int(), C.c_int()
    _check(load().operand_coords(shape, operand, lane, i, C.byref(r), C.byref(c)), "operand_coords")
    return r.value, c.value


def operand_offset(shape: int, operand: int, lane: int, i: int) -> int:
    o = C.c_int()
    _check(load().operand_offset(shape, operand, lane, i, C.byref(o)), "operand_offset")
    return o.value


def operand_decode(shape: int, operand: int, offset: int) -> Tuple[int, int]:
    lane, i = C.c_int(), C.c_int()
    _check(load().operand_decode(shape, operand, offset, C.byref(lane), C.byref(i)), "operand_decode")
    return lane.value, i.value


def operand_matrix_offset(shape: int, operand: int, lane: int, i: int, row0: int, col0: int, ld: int,
                          order: int) -> Optional[int]:
    """Strided source, or None when the library reports MFL_EOVERFLOW."""
    o = C.c_int64()
    st = load().operand_matrix_offset(shape, operand, lane, i, row0, col0, ld, order, C.byref(o))
    if st == EOVERFLOW:
        return None
    _check(st, "operand_matrix_offset")
    return o.value


def operand_load_strided(shape, operand, m, row0, col0, ld, order, frag, stream=None) -> None:
    info = _layout_info(load().mfl_operand_info, shape, operand)
    if info:  # an unknown shape or operand is left to the library to reject
        lanes, per_lane, rows, cols = info
        _need("operand_load_strided", m=(m, _op(row0 + rows, col0 + cols, ld, order, 2)),
              frag=(frag, lanes * per_lane * 2))
    _check(load().operand_load_strided(shape, operand, _ptr(m), row0, col0, ld, order, _ptr(frag), _stream(stream)),
           "operand_load_strided")


def acc_store_strided(shape, acc, c, row0, col0, ldc, stream=None) -> None:
    info = _layout_info(load().mfl_acc_info, shape)
    if info:
        lanes, per_lane, rows, cols = info
        _need("acc_store_strided", acc=(acc, lanes * per_lane * 4), c=(c, _extent(row0 + rows, col0 + cols, ldc, 4)))
    _check(load().acc_store_strided(shape, _ptr(acc), _ptr(c), row0, col0, ldc, _stream(stream)),
           "acc_store_strided")


def mfma_probe(shape, dtype, a_frag, b_frag, c_in, acc, stream=None) -> None:
    info = _layout_info(load().mfl_acc_info, shape)
    if info:
        lanes, per_lane, _, _ = info
        _need("mfma_probe", a_frag=(a_frag, 64 * 8 * 2), b_frag=(b_frag, 64 * 8 * 2),
              c_in=(c_in, lanes * per_lane * 4), acc=(acc, lanes * per_lane * 4))
    _check(load().mfma_probe(shape, dtype, _ptr(a_frag), _ptr(b_frag), _ptr(c_in), _ptr(acc), _stream(stream)),
           "mfma_probe")


RATE_PROBE_OUTPUTS = 2048 * 256   # MFL_RATE_PROBE_OUTPUTS


def mfma_rate_flops(iters: int) -> float:
    """Floating-point operations of one mfma_rate_probe call."""
    return RATE_PROBE_OUTPUTS // 64 * iters * 16 * 16384.0


def mfma_rate_probe(dtype, iters, seed, out, stream=None) -> None:
    _need("mfma_rate_probe", out=(out, RATE_PROBE_OUTPUTS * 4))
    _check(load().mfma_rate_probe(dtype, iters, seed, _ptr(out), _stream(stream)), "mfma_rate_probe")


def quantize_fp32(dtype, x, out, n, stream=None) -> None:
    _need("quantize_fp32", x=(x, max(n, 0) * 4), out=(out, max(n, 0) * 2))
    _check(load().quantize_fp32(dtype, _ptr(x), _ptr(out), n, _stream(stream)), "quantize_fp32")


def split_fp32(dtype, x, hi, lo, n, stream=None) -> None:
    _need("split_fp32", x=(x, max(n, 0) * 4), hi=(hi, max(n, 0) * 2), lo=(lo, max(n, 0) * 2))
    _check(load().split_fp32(dtype, _ptr(x), _ptr(hi), _ptr(lo), n, _stream(stream)), "split_fp32")


def gemm_tile_mma(dtype, m, n, k, a, lda, order_a, b, ldb, order_b, c, ldc, accumulate=0, stream=None) -> None:
    _need("gemm_tile_mma", a=(a, _op(m, k, lda, order_a, 2)), b=(b, _op(k, n, ldb, order_b, 2)),
          c=(c, _extent(m, n, ldc, 4)))
    _check(load().gemm_tile_mma(dtype, m, n, k, _ptr(a), lda, order_a, _ptr(b), ldb, order_b, _ptr(c), ldc,
                                accumulate, _stream(stream)), "gemm_tile_mma")


def gemm_tile_mma_shape(shape, dtype, m, n, k, a, lda, order_a, b, ldb, order_b, c, ldc, accumulate=0,
                        stream=None) -> None:
    _need("gemm_tile_mma_shape", a=(a, _op(m, k, lda, order_a, 2)), b=(b, _op(k, n, ldb, order_b, 2)),
          c=(c, _extent(m, n, ldc, 4)))
    _check(load().gemm_tile_mma_shape(shape, dtype, m, n, k, _ptr(a), lda, order_a, _ptr(b), ldb, order_b, _ptr(c),
                                      ldc, accumulate, _stream(stream)), "gemm_tile_mma_shape")


def gemm_block_repeat(dtype, tm, tn, tk, threads, repeats, m, n, a, b, c, stream=None) -> None:
    _need("gemm_block_repeat", a=(a, _extent(m, tk, tk, 2)), b=(b, _extent(n, tk, tk, 2)), c=(c, _extent(m, n, n, 4)))
    _check(load().gemm_block_repeat(dtype, tm, tn, tk, threads, repeats, m, n, _ptr(a), _ptr(b), _ptr(c),
                                    _stream(stream)), "gemm_block_repeat")


def gemm_block_repeat_lds_api(dtype, tm, tn, tk, threads, repeats, m, n, a, b, c, stream=None) -> None:
    _need("gemm_block_repeat_lds_api", a=(a, _extent(m, tk, tk, 2)), b=(b, _extent(n, tk, tk, 2)),
          c=(c, _extent(m, n, n, 4)))
    _check(load().gemm_block_repeat_lds_api(dtype, tm, tn, tk, threads, repeats, m, n, _ptr(a), _ptr(b), _ptr(c),
                                            _stream(stream)), "gemm_block_repeat_lds_api")


def gemm_split_fp32(piece, m, n, k, a, lda, order_a, mode_a, b, ldb, order_b, mode_b, chains, lolo, c, ldc,
                    accumulate=0, stream=None) -> None:
    _need("gemm_split_fp32", a=(a, _op(m, k, lda, order_a, 4)), b=(b, _op(k, n, ldb, order_b, 4)),
          c=(c, _extent(m, n, ldc, 4)))
    _check(load().gemm_split_fp32(piece, m, n, k, _ptr(a), lda, order_a, mode_a, _ptr(b), ldb, order_b, mode_b,
                                  chains, lolo, _ptr(c), ldc, accumulate, _stream(stream)), "gemm_split_fp32")


def gemm_split_fp32_workspace_bytes(m, n, k, lda, order_a, mode_a, ldb, order_b, mode_b, ldc) -> int:
    b = C.c_int64()
    _check(load().gemm_split_fp32_workspace_bytes(m, n, k, lda, order_a, mode_a, ldb, order_b, mode_b, ldc,
                                                  C.byref(b)), "gemm_split_fp32_workspace_bytes")
    return b.value


def gemm_split_fp32_ws(piece, m, n, k, a, lda, order_a, mode_a, b, ldb, order_b, mode_b, chains, lolo, c, ldc,
                       accumulate, workspace, workspace_bytes, stream=None) -> None:
    _need("gemm_split_fp32_ws", a=(a, _op(m, k, lda, order_a, 4)), b=(b, _op(k, n, ldb, order_b, 4)),
          c=(c, _extent(m, n, ldc, 4)), workspace=(workspace, max(workspace_bytes, 0)))
    _check(load().gemm_split_fp32_ws(piece, m, n, k, _ptr(a), lda, order_a, mode_a, _ptr(b), ldb, order_b, mode_b,
                                     chains, lolo, _ptr(c), ldc, accumulate, _ptr(workspace), workspace_bytes,
                                     _stream(stream)), "gemm_split_fp32_ws")


def attention_workspace_bytes(nq, nk, d, algo=1) -> int:
    b = C.c_int64()
    _check(load().attention_workspace_bytes(nq, nk, d, algo, C.byref(b)), "attention_workspace_bytes")
    return b.value


ATTN_STATIC_SCRATCH_BYTES = 64 << 20   # MFL_ATTN_STATIC_SCRATCH_BYTES


def attention_split_fp32_static(nq, nk, d, q, k, v, chains, algo, o, stream=None) -> None:
    _need("attention_split_fp32_static", q=(q, _extent(nq, d, d, 4)), k=(k, _extent(nk, d, d, 4)),
          v=(v, _extent(nk, d, d, 4)), o=(o, _extent(nq, d, d, 4)))
    _check(load().attention_split_fp32_static(nq, nk, d, _ptr(q), _ptr(k), _ptr(v), chains, algo, _ptr(o),
                                              _stream(stream)), "attention_split_fp32_static")


def attention_split_fp32(nq, nk, d, q, k, v, chains, algo, o, workspace, workspace_bytes, stream=None) -> None:
    _need("attention_split_fp32", q=(q, _extent(nq, d, d, 4)), k=(k, _extent(nk, d, d, 4)),
          v=(v, _extent(nk, d, d, 4)), o=(o, _extent(nq, d, d, 4)), workspace=(workspace, max(workspace_bytes, 0)))
    _check(load().attention_split_fp32(nq, nk, d, _ptr(q), _ptr(k), _ptr(v), chains, algo, _ptr(o),
                                       _ptr(workspace), workspace_bytes, _stream(stream)), "attention_split_fp32")
