"""ssd_forward_noalloc (through the C ABI) against ssd_forward with a
workspace, and against the fp64 oracle.

The entry point keeps g and dt_t in the library's per-GPU scratch array, so
two calls in a row reuse it: the second call here has a smaller input than
the first and must not see anything the first left behind.  Both entry
points launch the same kernels on the same inputs, so their outputs must be
equal bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, device_inputs, log
from ssd_workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _outputs(w, dev, y_dtype=torch.float32):
    b, L, H, P, N, nc = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.nchunks
    y = torch.full((b, L, H, P), float("nan"), device=DEV, dtype=y_dtype)
    states = torch.full((b, H, nc, P, N), float("nan"), device=DEV)
    final = torch.full((b, H, P, N), float("nan"), device=DEV)
    return y, states, final


def _both(ssd, w, seed):
    inp = make_inputs(w, seed=seed)
    dev = device_inputs(inp, w.dtype)
    T = w.chunk_size
    y1, s1, f1 = _outputs(w, dev)
    d = ssd.make_dims(dev["x"], dev["B"], T)
    ws = torch.empty(ssd.workspace_bytes(d), dtype=torch.uint8, device=DEV)
    ssd.ssd_forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"],
                    dev["init_state"], y1, s1, f1, ws, T)
    y2, s2, f2 = _outputs(w, dev)
    ssd.ssd_forward_noalloc(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"],
                            dev["init_state"], y2, s2, f2, T)
    torch.cuda.synchronize()
    return inp, (y1, s1, f1), (y2, s2, f2)


def test_noalloc_equals_forward_on_two_calls_in_a_row(ssd):
    big = Workload("noalloc_big", 4, 1000, 8, 64, 128, 2, 128, "bf16", -2.0, 0.0, 1.5, 0.1)
    small = Workload("noalloc_small", 1, 300, 4, 64, 64, 1, 64, "fp32", -1.0, -1.0, 2.0, None)
    for w, seed in ((big, 201), (small, 202)):
        log(f"[noalloc] {w}")
        inp, ref_outs, outs = _both(ssd, w, seed)
        for name, a, b in zip(("y", "states", "final"), ref_outs, outs):
            assert torch.equal(a, b), f"{w.name}: {name} differs from ssd_forward"
        ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                             inp["init_state"], chunk_size=w.chunk_size)
        y, states, final = (t.float().cpu().numpy() for t in outs)
        assert_close(states, ref["states"], w.dtype, "states")
        assert_close(final, ref["final"], w.dtype, "final")
        assert_close(y, ref["y"], w.dtype, "y")


def test_noalloc_rejects_shapes_past_its_scratch(ssd):
    # 8 * b * H * L bytes of g and dt_t must fit the per-GPU array; the check
    # runs on the host before any HIP call
    H = 64
    L = ssd.NOALLOC_SCRATCH_BYTES // 8 // H + 1
    x = torch.empty(1, L, H, 64, device=DEV, dtype=torch.bfloat16)
    B = torch.empty(1, L, 1, 64, device=DEV, dtype=torch.bfloat16)
    dt = torch.empty(1, L, H, device=DEV)
    A = torch.empty(H, device=DEV)
    y = torch.empty(1, L, H, 64, device=DEV)
    states = torch.empty(1, H, -(-L // 256), 64, 64, device=DEV)
    with pytest.raises(ssd.SsdError) as e:
        ssd.ssd_forward_noalloc(x, dt, A, B, B, A, None, y, states, None, 256)
    assert e.value.status == ssd.SSD_ERR_WORKSPACE
