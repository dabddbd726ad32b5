"""Helpers for the GPU parity tests: moving seeded inputs to the device as bf16
or float32 tensors, reading results back, and the error measures.

Tolerance reading (bf16 inputs, float32 accumulation): normwise max relative
error max|g - r| / max|r| <= 2e-2 and mean absolute error mean|g - r| <= 1e-3,
against the oracle in matched mode (bf16 rounding at the GPU's storage points).
float32 paths: normwise <= 1e-5. Byte/index work: bit-exact.
"""
import sys

import numpy as np
import torch

BF16_NORMWISE = 2e-2
BF16_MEAN_ABS = 1e-3
F32_NORMWISE = 1e-5

DEV = "cuda:0"


def note(msg):
    """Name the case before the GPU work starts (flushed, so a crash shows it)."""
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def f32_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def f64_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.detach().float().cpu().numpy().astype(np.float64)
    return t.detach().cpu().numpy().astype(np.float64)


def errors(g: np.ndarray, r: np.ndarray):
    d = np.abs(np.asarray(g, np.float64) - np.asarray(r, np.float64))
    scale = float(np.max(np.abs(r))) if r.size else 0.0
    return (float(d.max()) / scale if scale > 0 else float(d.max()) if d.size else 0.0,
            float(d.mean()) if d.size else 0.0)


def assert_bf16_close(g, r, what=""):
    rel, mae = errors(g, r)
    note(f"{what}: normwise {rel:.3e}, mean abs {mae:.3e}")
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert rel <= BF16_NORMWISE and mae <= BF16_MEAN_ABS, f"{what}: normwise {rel:.3e}, mean abs {mae:.3e}"
    return rel, mae


def assert_f32_close(g, r, what=""):
    rel, _ = errors(g, r)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    assert rel <= F32_NORMWISE, f"{what}: normwise {rel:.3e}"
    return rel
