"""Helpers for the GPU parity tests: device tensors from the seeded fp32
inputs, and the library's own quantisation to produce 16-bit device operands.

torch provides device memory and the stream; all arithmetic under test runs in
libmfl.so's kernels, reached through the ctypes binding."""
import sys

import numpy as np
import torch

import mma_fragment_layouts_amd as mfl

DT = {"f16": mfl.F16, "bf16": mfl.BF16}


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch.device("cuda:0")


def stream():
    return torch.cuda.current_stream()


def say(*args):
    """Name the case before a GPU step (flushed), so a failing run shows it."""
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def dev32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device())


def q16(x: np.ndarray, fmt: str) -> torch.Tensor:
    """16-bit device copy of fp32 values, rounded by the library's kernel."""
    src = dev32(x)
    out = torch.empty(src.shape, dtype=torch.int16, device=device())
    mfl.quantize_fp32(DT[fmt], src, out, src.numel(), stream())
    return out


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()
