"""Helpers for the GPU parity tests: device copies and tolerance checks.

Tolerances (stated per output: y, states, final):
* fp32 inputs: max |got - ref| / max(|ref|, RMS(ref)) <= 1e-4.
* bf16 inputs with fp32 y: max |got - ref| / RMS(ref) <= 2e-2, and a tighter
  bound of 2e-3 that the arithmetic itself supports (exact bf16 inputs,
  two-term bf16 splits of every computed operand, fp32 accumulation); the
  second bound catches a lost split term long before the first would.
* bf16 y (rounded output): RMS-floored relative error <= 1e-2 (the final
  rounding alone is 2^-9 relative to each element).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from closed_forms import rel_err, rms_err

FP32_TOL = 1e-4
BF16_TOL = 2e-2
BF16_ARITH_TOL = 2e-3
BF16_Y_TOL = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def device_inputs(inp, dtype: str, device="cuda:0"):
    """numpy inputs -> device tensors (x, B, C in the storage dtype)."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    out = {}
    for k in ("x", "B", "C"):
        out[k] = torch.from_numpy(inp[k]).to(device=device, dtype=tdt).contiguous()
    for k in ("dt", "A", "D"):
        out[k] = torch.from_numpy(inp[k]).to(device).contiguous()
    init = inp.get("init_state")
    out["init_state"] = (None if init is None
                         else torch.from_numpy(np.ascontiguousarray(init, np.float32)).to(device))
    return out


def assert_close(got, ref, dtype: str, what: str, y_bf16: bool = False):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    if y_bf16:
        e = rel_err(got, ref)
        log(f"  {what}: rel(RMS-floored)={e:.3e}")
        assert e <= BF16_Y_TOL, (what, e)
    elif dtype == "fp32":
        e = rel_err(got, ref)
        log(f"  {what}: rel(RMS-floored)={e:.3e}")
        assert e <= FP32_TOL, (what, e)
    else:
        e = rms_err(got, ref)
        log(f"  {what}: max|d|/RMS={e:.3e}")
        assert e <= BF16_TOL, (what, e)
        assert e <= BF16_ARITH_TOL, (what, e)
    return e


def g_tolerance(g_ref: np.ndarray, T: int) -> np.ndarray:
    """Bound for the fp32 stage-1 result: each product, each of the T
    same-signed additions and the final scaling round once, so
    |err| <= (T + 3) 2^-24 |g| (A dt <= 0 keeps the partial sums monotone)."""
    return (T + 3) * 2.0 ** -24 * np.abs(g_ref) + 1e-30
