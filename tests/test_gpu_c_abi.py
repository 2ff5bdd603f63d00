"""The C ABI used from a plain C99 program on the device (tests/c/abi_device_gemm.c):
device rounding and the tiled GEMM called without Python, results checked on
sampled entries against a double-precision dot product of the rounded values,
C's padding column checked untouched."""
import shutil
import subprocess

import pytest

from test_abi_host import device_program_command

pytestmark = pytest.mark.gpu


def test_c_program_runs_the_gemm_on_the_device(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler on this host")
    exe = tmp_path / "abi_device_gemm"
    build = subprocess.run(device_program_command(cc, exe), capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    print("[gpu] C program: abi_device_gemm", flush=True)
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    print(run.stdout)
    assert run.returncode == 0, run.stderr
    assert "abi_device_gemm: ok" in run.stdout
