"""Parity of the streaming decode step (ssd_decode_step, through the C ABI)
with the fp64 oracle.

One decode step is the recurrence over a single token with the carried state
as the initial state, so the oracle's forward pass over the same tokens is
its reference: one step, many steps in a row (each step's y and the state
after the last), and steps that continue a sequence after a prefill run by
ssd_forward.  The step's arithmetic is fp32 throughout (bf16 inputs are exact
values), so single steps are held to the fp32 tolerance for either input
type.
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


def _wl(dtype, b, L, H, G, N, init=True, T=64):
    return Workload(f"decode_{dtype}", b, L, H, 64, N, G, T, dtype, -2.0, 0.0,
                    1.5, 0.5 if init else None)


def _np(t):
    return t.detach().float().cpu().numpy()


def _token(dev, t):
    """Token t of the forward-pass tensors, in the decode-step layouts."""
    return (dev["x"][:, t].contiguous(), dev["dt"][:, t].contiguous(),
            dev["B"][:, t].contiguous(), dev["C"][:, t].contiguous())


CASES = [
    ("bf16", 3, 5, 4, 2, 128),
    ("bf16", 2, 5, 6, 3, 64),
    ("fp32", 2, 5, 4, 1, 128),
    ("fp32", 4, 5, 6, 6, 64),
    # enough (b, h) pairs for two and for one workgroup per head
    ("bf16", 4, 2, 64, 2, 128),
    ("fp32", 8, 2, 64, 4, 64),
]


@pytest.mark.parametrize("dtype,b,L,H,G,N", CASES,
                         ids=[f"{c[0]}_b{c[1]}_H{c[3]}_G{c[4]}_N{c[5]}" for c in CASES])
def test_decode_steps_match_recurrence(ssd, dtype, b, L, H, G, N):
    """L decode steps from a random state equal the oracle's forward over the
    L tokens with that state as init_state: every step's y, and the state
    after the last step."""
    w = _wl(dtype, b, L, H, G, N)
    inp = make_inputs(w, seed=41)
    log(f"[decode] {dtype} b={b} L={L} H={H} G={G} N={N}")
    dev = device_inputs(inp, dtype)
    state = dev["init_state"].clone()
    ys = []
    for t in range(L):
        xt, dtt, Bt, Ct = _token(dev, t)
        y = torch.empty(b, H, 64, device=DEV)
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], state, y)
        ys.append(y)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    got_y = np.stack([_np(y) for y in ys], axis=1)      # [b, L, H, P]
    assert_close(got_y, ref["y"], "fp32", "decode y")
    assert_close(_np(state), ref["final"], "fp32", "decode state")


def test_decode_continues_a_prefill(ssd):
    """ssd_forward over the first tokens, then decode steps from its final
    state: the outputs continue the oracle's run over all tokens."""
    w = _wl("bf16", 2, 200, 4, 1, 128, init=False)
    inp = make_inputs(w, seed=42)
    dev = device_inputs(inp, "bf16")
    L0 = 197
    pre = {k: (v[:, :L0].contiguous() if k in ("x", "dt", "B", "C") else v)
           for k, v in dev.items()}
    _, _, final = ssd.forward(pre["x"], pre["dt"], pre["A"], pre["B"], pre["C"],
                              pre["D"], None, chunk_size=64)
    state = final.clone()
    ys = []
    for t in range(L0, w.seqlen):
        xt, dtt, Bt, Ct = _token(dev, t)
        y = torch.empty(w.batch, w.nheads, 64, device=DEV)
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], state, y)
        ys.append(y)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], None, chunk_size=64)
    got_y = np.stack([_np(y) for y in ys], axis=1)
    # the carried state holds the prefill's bf16-path error, so the bf16 bound
    assert_close(got_y, ref["y"][:, L0:], "bf16", "y after prefill")
    assert_close(_np(state), ref["final"], "bf16", "state after prefill")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_zero_dt_keeps_state_exactly(ssd, dtype):
    """dt = 0: exp(0) = 1 and the input term vanishes, so the state is
    unchanged bit for bit and y = state C + D x."""
    w = _wl(dtype, 2, 1, 4, 2, 128)
    inp = make_inputs(w, seed=43)
    inp["dt"] = np.zeros_like(inp["dt"])
    dev = device_inputs(inp, dtype)
    state = dev["init_state"].clone()
    xt, dtt, Bt, Ct = _token(dev, 0)
    y = torch.empty(2, 4, 64, device=DEV)
    ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], state, y)
    torch.cuda.synchronize()
    assert torch.equal(state, dev["init_state"])
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=64)
    assert_close(_np(y)[:, None], ref["y"], "fp32", "y with dt = 0")


def test_decode_bf16_output(ssd):
    w = _wl("bf16", 2, 1, 4, 1, 64)
    inp = make_inputs(w, seed=44)
    dev = device_inputs(inp, "bf16")
    state = dev["init_state"].clone()
    xt, dtt, Bt, Ct = _token(dev, 0)
    y = torch.empty(2, 4, 64, device=DEV, dtype=torch.bfloat16)
    ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], state, y)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=64)
    assert_close(_np(y)[:, None], ref["y"], "bf16", "bf16 y", y_bf16=True)


def test_decode_binding_rejects_bad_arguments(ssd):
    w = _wl("bf16", 2, 1, 4, 2, 128)
    dev = device_inputs(make_inputs(w, seed=45), "bf16")
    xt, dtt, Bt, Ct = _token(dev, 0)
    state = dev["init_state"].clone()
    y = torch.empty(2, 4, 64, device=DEV)
    with pytest.raises(ValueError):
        ssd.ssd_decode_step(xt, dtt[:, :-1].contiguous(), dev["A"], Bt, Ct,
                            dev["D"], state, y)
    with pytest.raises(TypeError):
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt.float(), Ct, dev["D"], state, y)
    with pytest.raises(ssd.SsdError):
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt[:, :, :96].contiguous(),
                            Ct[:, :, :96].contiguous(), dev["D"],
                            state[..., :96].contiguous(), y)


def test_decode_step_replays_from_a_hip_graph(ssd):
    """One decode step captured in a HIP graph and replayed several times
    (with eager work and synchronisations in between) advances the state
    exactly as the same number of eager steps does."""
    w = _wl("bf16", 2, 1, 4, 2, 128)
    dev = device_inputs(make_inputs(w, seed=46), "bf16")
    xt, dtt, Bt, Ct = _token(dev, 0)
    eager_state = dev["init_state"].clone()
    graph_state = dev["init_state"].clone()
    y_eager = torch.empty(2, 4, 64, device=DEV)
    y_graph = torch.empty(2, 4, 64, device=DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], graph_state, y_graph)
    torch.cuda.synchronize()
    # capture only records: the state is still the initial one
    assert torch.equal(graph_state, dev["init_state"])
    for rep in range(4):
        ssd.ssd_decode_step(xt, dtt, dev["A"], Bt, Ct, dev["D"], eager_state, y_eager)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(graph_state, eager_state), rep
        assert torch.equal(y_graph, y_eager), rep
