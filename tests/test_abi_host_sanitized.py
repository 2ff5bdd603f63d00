"""The host side of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.

The argument validation, size and workspace arithmetic and dispatch decisions
of every entry point run on the host before any HIP call; this test rebuilds the
library with its host code instrumented (``build(sanitize=True)``: the device
code is unchanged), loads that build into a fresh Python process with the ASan
runtime preloaded, and runs the whole host ABI suite (tests/test_abi_host.py)
against it.  Any out-of-bounds access, use after free, signed overflow or
other undefined behaviour on those paths fails the run."""
import glob
import os
import subprocess
import sys

from mma_fragment_layouts_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _sanitized_library() -> str:
    deps = B.sources() + glob.glob(os.path.join(B.CSRC, "*.hpp")) + [os.path.join(ROOT, "include", "mfl.h")]
    if not os.path.exists(B.LIB_SAN) or any(os.path.getmtime(d) > os.path.getmtime(B.LIB_SAN) for d in deps):
        B.build(sanitize=True, verbose=False)
    return B.LIB_SAN


def _env(lib):
    return dict(os.environ, MFL_LIBRARY=lib, LD_PRELOAD=B.sanitizer_runtime(), ASAN_OPTIONS="detect_leaks=0",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def test_host_abi_suite_under_asan_and_ubsan():
    lib = _sanitized_library()
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in undefined and "__ubsan_handle" in undefined, "host code is not instrumented"
    # the child process maps the instrumented build, not the default one
    probe = ("import mma_fragment_layouts_amd as m; m.load(); "
             "print(any(l.rstrip().endswith('libmfl_san.so') for l in open('/proc/self/maps')))")
    r = subprocess.run([sys.executable, "-c", probe], env=_env(lib), capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0 and r.stdout.strip() == "True", r.stdout + r.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-k", "not plain_c",
                        os.path.join(ROOT, "tests", "test_abi_host.py")], env=_env(lib), capture_output=True,
                       text=True, timeout=900, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " passed" in r.stdout
