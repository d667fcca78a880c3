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


def compare_all_pairs(fetch_ref, fetch_got, npairs: int, per_batch: int, dtype: str,
                      names, label: str = ""):
    """Compare every element of the named outputs over all (batch, head)
    pairs, `per_batch` pairs at a time so host memory stays bounded.

    fetch_ref(p0, p1) and fetch_got(p0, p1) return dicts name -> array whose
    first axis is the pairs p0 .. p1-1 (pair = b * nheads + h).  The
    tolerances are those of ``assert_close``, normalised by the RMS of the
    whole reference output: a first pass over the oracle accumulates it, a
    second pass takes the errors.
    """
    bounds = [(p0, min(p0 + per_batch, npairs)) for p0 in range(0, npairs, per_batch)]
    ss = {n: 0.0 for n in names}
    cnt = {n: 0 for n in names}
    for p0, p1 in bounds:
        ref = fetch_ref(p0, p1)
        for n in names:
            r = np.asarray(ref[n], np.float64)
            ss[n] += float(np.sum(r * r))
            cnt[n] += r.size
        del ref
    rms = {n: (ss[n] / cnt[n]) ** 0.5 if cnt[n] else 0.0 for n in names}
    worst = {n: 0.0 for n in names}
    for p0, p1 in bounds:
        ref = fetch_ref(p0, p1)
        got = fetch_got(p0, p1)
        for n in names:
            r = np.asarray(ref[n], np.float64)
            gv = np.asarray(got[n], np.float64)
            assert gv.shape == r.shape, (n, gv.shape, r.shape)
            assert np.all(np.isfinite(gv)), f"{label}{n}: non-finite values in pairs {p0}..{p1 - 1}"
            d = np.abs(gv - r)
            if dtype == "fp32":
                den = np.maximum(np.abs(r), rms[n])
                den = np.where(den == 0, 1.0, den)
                e = float(np.max(d / den)) if d.size else 0.0
            else:
                e = float(np.max(d)) / rms[n] if rms[n] > 0 else float(np.max(d))
            worst[n] = max(worst[n], e)
        del ref, got
    for n in names:
        e = worst[n]
        if dtype == "fp32":
            log(f"  {label}{n} (all {npairs} pairs): rel(RMS-floored)={e:.3e}")
            assert e <= FP32_TOL, (n, e)
        else:
            log(f"  {label}{n} (all {npairs} pairs): max|d|/RMS={e:.3e}")
            assert e <= BF16_TOL, (n, e)
            assert e <= BF16_ARITH_TOL, (n, e)
    return worst


def pairs_per_batch(w, budget_bytes: float = 1.0e9) -> int:
    """Pairs whose fp64 oracle outputs (y and states) fit in about
    `budget_bytes` of host memory."""
    per = 8 * (w.seqlen * w.headdim + w.nchunks * w.headdim * w.dstate)
    return max(1, int(budget_bytes // per))
