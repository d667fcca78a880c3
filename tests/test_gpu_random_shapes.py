"""ssd_forward against the fp64 oracle over a seeded draw of shapes.

The named cases elsewhere pick the shapes that select each kernel path; this
module adds breadth: 32 shapes drawn once from a fixed seed over every
supported combination (batch 1-3, 1-700 tokens, 1-12 heads with any group
count dividing them, N in {64, 128}, T in {64, 128, 256}, bf16 or fp32
inputs, with or without an initial state, fp32 or bf16 y).  Each is compared
element by element at the tolerances of the parity suite.  The draw is made
here, from its own generator, so the list is the same on every run.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, device_inputs, log
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _draw(n=32, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 13))
        divisors = [g for g in range(1, H + 1) if H % g == 0]
        G = int(rng.choice(divisors))
        T = int(rng.choice([64, 128, 256]))
        L = int(rng.integers(1, 701))
        b = int(rng.integers(1, 4))
        N = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp32"]))
        init = bool(rng.integers(0, 2))
        ybf16 = bool(rng.integers(0, 4) == 0)
        out.append((i, b, L, H, G, N, T, dtype, init, ybf16))
    return out


CASES = _draw()


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "r%02d_b%d_L%d_H%d_G%d_N%d_T%d_%s%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], "_init" if c[8] else "", "_ybf16" if c[9] else ""))
def test_random_shape(ssd, case):
    i, b, L, H, G, N, T, dtype, init, ybf16 = case
    w = Workload("random", b, L, H, 64, N, G, T, dtype, -2.0, 0.0, 1.5, 0.1 if init else None)
    log(f"[random] {case}")
    inp = make_inputs(w, seed=500 + i)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T)
    dev = device_inputs(inp, dtype)
    y, states, final = ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"],
                                   dev["D"], dev["init_state"], chunk_size=T,
                                   y_dtype=torch.bfloat16 if ybf16 else torch.float32)
    torch.cuda.synchronize()
    assert_close(_np(states), ref["states"], dtype, "states")
    assert_close(_np(final), ref["final"], dtype, "final")
    assert_close(_np(y), ref["y"], dtype, "y", y_bf16=ybf16)
