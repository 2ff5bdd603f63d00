"""Builds libmfl.so in-tree with hipcc for gfx950.

Every ``csrc/*.hip`` file is compiled to an object under ``_build/`` (in
parallel) and the objects are linked into ``lib/libmfl.so`` next to this file.
Run ``python -m mma_fragment_layouts_amd.build`` or call ``build()``.

``build(sanitize=True)`` (``--sanitize``) makes a second library,
``_build_san/libmfl_san.so``, whose host code is instrumented with
AddressSanitizer and UndefinedBehaviorSanitizer (the device code is built as
usual): the argument validation, workspace arithmetic and dispatch of the C ABI
run under the sanitizers on a CPU-only machine.  It needs the ASan runtime
preloaded (see ``sanitizer_runtime()``).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "lib", "libmfl.so")
ARCH = os.environ.get("MFL_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-Wall", "-Wno-unused-function",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators and results in the architectural VGPRs.  Left to itself
    # the compiler splits a large accumulator set between VGPRs and AGPRs and
    # copies it back and forth around the MFMAs (hundreds of v_accvgpr moves per
    # loop in the 128 x 128 GEMM tiles and the block-repeat tiles); with this form
    # the 128 x 128 block-repeat kernel runs 28 % faster and the 64 x 64 ones
    # 13-22 %, and kernels whose registers fit either way compile to the same code.
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
]


OBJ_SAN = os.path.join(HERE, "_build_san")
LIB_SAN = os.path.join(OBJ_SAN, "libmfl_san.so")
# host code only: each -fsanitize= goes right after -Xarch_host
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined"]


def sanitizer_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that an uninstrumented
    program (python) must preload to load libmfl_san.so."""
    out = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    return out.stdout.strip()


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(OBJ_SAN if sanitize else OBJ, os.path.basename(src)[:-4] + ".o")
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS if sanitize else FLAGS
    cmd = [HIPCC, *flags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int | None = None, verbose: bool = True, sanitize: bool = False) -> str:
    out = LIB_SAN if sanitize else LIB
    os.makedirs(OBJ_SAN if sanitize else OBJ, exist_ok=True)
    os.makedirs(os.path.dirname(out), exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), srcs))
    tmp = out + ".tmp"
    link_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_san, *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv)
