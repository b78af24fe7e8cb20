"""Helpers for the GPU parity tests: host <-> device transfers of bf16 bit
patterns and byte tensors.  No method arithmetic."""
from __future__ import annotations

import numpy as np
import pytest
import torch

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(),
                                  reason="needs an MI355X GPU")


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> device bfloat16 tensor (same bytes)."""
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    idx = np.argwhere(a != b)
    if idx.size == 0:
        return "equal"
    i = tuple(idx[0])
    return f"{len(idx)} mismatches; first at {i}: got {a[i]!r} want {b[i]!r}"


def assert_bytes_equal(got: np.ndarray, want: np.ndarray, what: str):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        raise AssertionError(f"{what}: {first_mismatch(got, want)}")


def gpu_normal_bf16(rows: int, cols: int, std: float, seed: int) -> torch.Tensor:
    """bf16 [rows, cols] N(0, std^2) drawn on the GPU from a seeded torch
    generator (for weight sets too large to draw on the host quickly)."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    out = torch.empty((rows, cols), dtype=torch.bfloat16, device="cuda")
    step = 1 << 16
    for r in range(0, rows, step):
        n = min(step, rows - r)
        out[r:r + n] = (torch.randn(n, cols, generator=g, device="cuda") * std).to(torch.bfloat16)
    return out
