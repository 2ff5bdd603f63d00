"""MFMA fragment layouts and tiled mixed-precision GEMMs for MI355X (gfx950).

The compute lives in ``lib/libmfl.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/mfl.h``); this package is its thin ctypes binding,
with the same function names, plus the seeded synthetic input generator
(``inputs``) and the in-tree build script (``build``).  Device memory and
streams come from the caller (e.g. torch tensors' ``data_ptr()`` and
``torch.cuda.current_stream()``).
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (EXPORTS, LIB_PATH, MflError, load, library_path,  # noqa: F401
                       status_string)
