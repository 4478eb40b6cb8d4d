"""Helpers shared by the GPU parity tests."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from block_scaled_fp4_05_amd import moe_fp4
    moe_fp4.lib()  # raises if the HIP library was not built: no silent fallback


def say(msg: str):
    """Name the case before a GPU step, flushed, so a failing run shows where it was."""
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def bf16_bits_of(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


TOL = 2e-3  # per-row relative L2 error bound of the grouped GEMM
