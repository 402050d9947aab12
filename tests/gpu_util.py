"""Helpers shared by the GPU tests: move storage-form numpy arrays to the device
and back, and the acceptance rules for floating-point results."""
import os
import sys

import numpy as np
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from sparse_hybrid_attention_amd import binding  # noqa: E402

DEV = "cuda:0"
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2
F32_ATOL = 1e-4


def lib():
    """Load the built library (builds it first only when nothing is built)."""
    if not os.path.exists(binding.LIB_PATH):
        from sparse_hybrid_attention_amd import build_lib
        build_lib.build()
    return binding.load_library()


def dev(a: np.ndarray, dtype: int = None) -> torch.Tensor:
    """Storage-form numpy array -> device tensor (uint16 bit patterns -> bfloat16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> storage-form numpy array."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def assert_close(got: np.ndarray, want: np.ndarray, what: str = ""):
    """fp32: max |got - want| <= 1e-4; bf16: |got - want| <= 2e-2 + 1e-2 |want|."""
    assert got.shape == want.shape, (got.shape, want.shape)
    g, w = as_f64(got), as_f64(want)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - w)
    if got.dtype == np.uint16:
        bad = err > BF16_ATOL + BF16_RTOL * np.abs(w)
        if bad.any():
            i = np.argwhere(bad)[0]
            raise AssertionError(f"{what}: {bad.sum()} elements outside bf16 tolerance; first at "
                                 f"{tuple(i)} got {g[tuple(i)]} want {w[tuple(i)]}")
    else:
        mx = err.max() if err.size else 0.0
        assert mx <= F32_ATOL, f"{what}: max abs err {mx} > {F32_ATOL}"
    return float(err.max()) if err.size else 0.0
