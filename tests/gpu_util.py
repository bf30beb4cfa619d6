"""Helpers of the GPU parity tests (marshalling and comparison only)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a HIP device (run them with -m gpu on an MI355X)")


def banner(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault can be traced."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def host_u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


def host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def assert_f32_close(got: np.ndarray, want: np.ndarray, rtol: float = 1e-6, scale=None, what=""):
    """|got - want| <= rtol * max(|want|, scale) elementwise (scale: an optional
    per-element magnitude floor, e.g. the operands of a sum)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    ref = np.abs(want) if scale is None else np.maximum(np.abs(want), np.asarray(scale, dtype=np.float64))
    with np.errstate(invalid="ignore"):
        bad = ~((got == want) | (np.abs(got - want) <= rtol * ref))
    bad &= ~(np.isnan(got) & np.isnan(want))
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements outside rtol={rtol}; first {idx.tolist()} "
                             f"got {got[tuple(idx.T)]} want {want[tuple(idx.T)]}")


def exact_fraction(got: np.ndarray, want: np.ndarray) -> float:
    g = np.asarray(got, dtype=np.float32).view(np.uint32)
    w = np.asarray(want, dtype=np.float32).view(np.uint32)
    return float((g == w).mean()) if g.size else 1.0
