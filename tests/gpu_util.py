"""Shared helpers of the GPU tests (not collected as tests)."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import kv_cache_attention_kvc_amd as kvc  # noqa: E402

TOL = {"f32": 1e-5, "f16": 2e-3, "e4m3": 3e-2, "i8": 3e-2}
NP = {"f32": np.float32, "f16": np.float16}
TD = {"f32": torch.float32, "f16": torch.float16}


def scale_of(D: int) -> float:
    """The fp32 scale 1/sqrt(D), passed identically to the kernels and the oracle."""
    return float(np.float32(1.0 / np.sqrt(D)))


def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kvc.load_library()
    return torch.device("cuda:0")


def to_dev(a, d):
    return torch.from_numpy(np.ascontiguousarray(a)).to(d)


def note(msg: str) -> None:
    """Print what the next GPU step is, flushed, so a failed run names its case."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def max_err(got, want) -> float:
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape
    assert np.isfinite(got).all(), "non-finite output"
    return float(np.abs(got - want).max()) if got.size else 0.0


def check(got, want, tol: float, what: str = "") -> float:
    """Max-abs error of got vs want, asserted <= tol with a short message."""
    err = max_err(got, want)
    if not err <= tol:
        raise AssertionError(f"{what}: max-abs error {err:.3e} > {tol:.1e}")
    return err
