"""Parity of the causal depthwise conv1d (ssd_causal_conv1d, through the C ABI)
with the fp64 oracle, element by element.

Tolerance, from the arithmetic: the kernel adds the W products onto the bias
with fp32 fused multiply-adds, so each output differs from the exact sum by
at most (W + 1) 2^-24 S, S = |bias| + sum_k |w_k x_(t-W+1+k)| (the oracle
evaluates S from the absolute values).  A bf16 output adds its rounding,
at most 2^-8 of the fp32 value.  The tests allow (W + 2) 2^-24 S, plus
2^-8 (|ref| + that) for bf16 output.

Cases cover both kernels (rows whose byte length is a multiple of 16 take
the vector kernel, others the per-token one), runs of several wavefronts
per row (the left neighbour at a run boundary), ragged runs at the row end,
rows shorter than the filter, every width 1..4, no bias, and the conv that
feeds the small-model Mamba-2 layer at full size (b 4, dim 1792, L 2048).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import log
from ssd_workloads import (WORKLOADS, ConvWorkload, conv_workload_for,
                           make_conv_inputs)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "fp32": torch.float32}


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _run(ssd, inp, xdt, odt):
    x = torch.from_numpy(inp["x"]).to(device=DEV, dtype=TDT[xdt]).contiguous()
    w = torch.from_numpy(inp["weight"]).to(DEV).contiguous()
    b = None if inp["bias"] is None else torch.from_numpy(inp["bias"]).to(DEV)
    out = torch.full(tuple(x.shape), float("nan"), device=DEV, dtype=TDT[odt])
    ssd.ssd_causal_conv1d(x, w, b, out)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64)


def _check(got, inp, odt, what):
    x, w, b = inp["x"], inp["weight"], inp["bias"]
    ref = oracle.causal_conv1d(x, w, b)
    S = oracle.causal_conv1d(np.abs(x), np.abs(w), None if b is None else np.abs(b))
    W = w.shape[1]
    bound = (W + 2) * 2.0 ** -24 * S
    if odt == "bf16":
        bound = bound + 2.0 ** -8 * (np.abs(ref) + bound)
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = np.abs(got - ref)
    worst = float(np.max(err / (bound + 1e-300)))
    log(f"  {what}: max|d|={err.max():.3e}  max|d|/bound={worst:.3f}")
    assert np.all(err <= bound), (what, worst)


CASES = [
    # xdt, odt, b, dim, L, W, bias
    ("bf16", "bf16", 2, 5, 2048, 4, True),    # one run per row (vector)
    ("bf16", "fp32", 2, 3, 4096, 4, True),    # two runs per row
    ("bf16", "bf16", 1, 4, 2056, 3, True),    # ragged second run
    ("bf16", "bf16", 3, 7, 40, 2, False),     # run much longer than the row
    ("bf16", "fp32", 2, 3, 1000, 4, True),    # L % 8 = 0, 125 units
    ("bf16", "bf16", 2, 3, 1001, 4, True),    # per-token kernel
    ("bf16", "bf16", 2, 6, 3, 4, True),       # shorter than the filter
    ("fp32", "fp32", 2, 5, 2048, 4, True),    # eight runs per row
    ("fp32", "bf16", 2, 3, 1028, 3, True),    # ragged last run
    ("fp32", "fp32", 1, 4, 1030, 4, False),   # per-token kernel
    ("fp32", "fp32", 3, 2, 1, 4, True),       # one token
    ("bf16", "bf16", 2, 4, 512, 1, True),     # width 1: no neighbour
    ("fp32", "fp32", 2, 4, 256, 2, True),
]


@pytest.mark.parametrize(
    "xdt,odt,b,dim,L,W,bias", CASES,
    ids=[f"{c[0]}_to_{c[1]}_b{c[2]}_d{c[3]}_L{c[4]}_W{c[5]}" + ("" if c[6] else "_nobias")
         for c in CASES])
def test_conv_matches_oracle(ssd, xdt, odt, b, dim, L, W, bias):
    c = ConvWorkload("conv_case", b, dim, L, W, xdt, bias)
    inp = make_conv_inputs(c, seed=100 + L + W)
    log(f"[conv] {xdt}->{odt} b={b} dim={dim} L={L} W={W} bias={bias}")
    _check(_run(ssd, inp, xdt, odt), inp, odt, "conv out")


@pytest.mark.parametrize("odt", ["bf16", "fp32"])
def test_conv_small_layer_full_size(ssd, odt):
    """The conv that feeds the small-model layer, at full size, launched as
    the benchmark launches it; every output is compared."""
    c = conv_workload_for(WORKLOADS["small_bf16"])
    inp = make_conv_inputs(c, seed=7)
    log(f"[conv] full size {c} -> {odt}")
    _check(_run(ssd, inp, c.dtype, odt), inp, odt, "conv full")


@pytest.mark.parametrize("xdt,t0", [("bf16", 2047), ("fp32", 255)])
def test_conv_impulse_places_taps(ssd, xdt, t0):
    """A unit impulse on the last token of a wavefront's run (2048 bf16 or
    256 fp32 tokens): the taps land in reverse order on the impulse and the
    W-1 tokens after it, in every row independently."""
    b, dim, L, W = 1, 3, 4096, 4
    x = np.zeros((b, dim, L), np.float32)
    x[0, :, t0] = 1.0
    w = np.arange(1, dim * W + 1, dtype=np.float32).reshape(dim, W)
    inp = {"x": x, "weight": w, "bias": None}
    got = _run(ssd, inp, xdt, "fp32")
    expect = np.zeros_like(got)
    for j in range(W):
        expect[0, :, t0 + j] = w[:, W - 1 - j]
    assert np.array_equal(got, expect)


def test_conv_rejects_bad_arguments(ssd):
    x = torch.zeros(2, 4, 64, device=DEV, dtype=torch.bfloat16)
    w = torch.zeros(4, 4, device=DEV)
    out = torch.empty_like(x)
    with pytest.raises(ValueError):
        ssd.ssd_causal_conv1d(x, w[:3].contiguous(), None, out)
    with pytest.raises(TypeError):
        ssd.ssd_causal_conv1d(x, w.bfloat16(), None, out)
    with pytest.raises(ssd.SsdError):
        ssd.ssd_causal_conv1d(x, torch.zeros(4, 5, device=DEV), None, out)
