"""Parity of the two-level state pass (ssd_chunk_state then
ssd_state_passing, through the C ABI) with the fp64 oracle.

* The two calls in sequence give the states and final state of the
  recurrence (bf16 tolerances of the parity suite), over ragged chunks,
  grouped B/C, an initial state, every chunk size and both state sizes.
* chunk_state alone: each chunk's contribution from a zero state equals the
  oracle's final state over that chunk alone, with a zero initial state.
* state_passing alone: fed the oracle's per-chunk contributions, it rebuilds
  the oracle's states at the fp32 tolerance (its arithmetic is fp32 only).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, compare_all_pairs, device_inputs, log
from ssd_workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _wl(b, L, H, G, N, T, init, dtype="bf16"):
    return Workload("two_level", b, L, H, 64, N, G, T, dtype, -2.0, 0.0, 1.5,
                    0.1 if init else None)


def _np(t):
    return t.detach().float().cpu().numpy()


def _cumsum(ssd, dev, w):
    b, L, H = w.batch, w.seqlen, w.nheads
    g = torch.empty(b, H, L, device=DEV)
    dtt = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dtt, w.chunk_size)
    return g, dtt


def _two_level(ssd, dev, w, g, dtt, with_final=True):
    b, H, P, N, nc = w.batch, w.nheads, w.headdim, w.dstate, w.nchunks
    states = torch.full((b, H, nc, P, N), float("nan"), device=DEV)
    fin = torch.full((b, H, P, N), float("nan"), device=DEV) if with_final else None
    ssd.ssd_chunk_state(dev["x"], dev["B"], dtt, g, states, fin, w.chunk_size)
    ssd.ssd_state_passing(g, dev["init_state"], states, fin, w.chunk_size)
    torch.cuda.synchronize()
    return states, fin


CASES = [
    # b, L, H, G, N, T, init
    (2, 300, 4, 2, 128, 64, True),
    (1, 700, 3, 1, 64, 256, False),
    (2, 333, 2, 1, 128, 128, True),
    (3, 37, 2, 1, 64, 64, False),       # shorter than a chunk
    (1, 1, 2, 2, 128, 128, True),       # one token
    (2, 450, 6, 3, 64, 64, True),
    (2, 4096, 8, 2, 128, 64, True),     # two heads per chunk_state workgroup
    (2, 8170, 8, 2, 64, 64, False),     # two heads per workgroup, ragged
    (1, 16384, 16, 1, 64, 256, False),  # two heads, 256-token chunks
]


@pytest.mark.parametrize("b,L,H,G,N,T,init", CASES,
                         ids=[f"b{c[0]}_L{c[1]}_H{c[2]}_G{c[3]}_N{c[4]}_T{c[5]}" + ("_init" if c[6] else "")
                              for c in CASES])
def test_two_level_matches_oracle(ssd, b, L, H, G, N, T, init):
    w = _wl(b, L, H, G, N, T, init)
    inp = make_inputs(w, seed=90 + L)
    log(f"[two-level] {w}")
    dev = device_inputs(inp, "bf16")
    g, dtt = _cumsum(ssd, dev, w)
    states, fin = _two_level(ssd, dev, w, g, dtt)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T, want_y=False)
    assert_close(_np(states), ref["states"], "bf16", "states")
    assert_close(_np(fin), ref["final"], "bf16", "final")


FP32_CASES = [
    # b, L, H, G, N, T, init: fp32 inputs (chunk_state's fp32 kernel)
    (2, 300, 4, 2, 128, 64, True),
    (1, 700, 3, 1, 64, 256, False),
    (2, 333, 2, 1, 128, 128, True),
    (3, 37, 2, 1, 64, 64, False),
]


@pytest.mark.parametrize("b,L,H,G,N,T,init", FP32_CASES,
                         ids=[f"fp32_b{c[0]}_L{c[1]}_H{c[2]}_G{c[3]}_N{c[4]}_T{c[5]}" + ("_init" if c[6] else "")
                              for c in FP32_CASES])
def test_two_level_fp32_matches_oracle(ssd, b, L, H, G, N, T, init):
    w = _wl(b, L, H, G, N, T, init, "fp32")
    inp = make_inputs(w, seed=190 + L)
    log(f"[two-level fp32] {w}")
    dev = device_inputs(inp, "fp32")
    g, dtt = _cumsum(ssd, dev, w)
    states, fin = _two_level(ssd, dev, w, g, dtt)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T, want_y=False)
    assert_close(_np(states), ref["states"], "fp32", "states")
    assert_close(_np(fin), ref["final"], "fp32", "final")


def test_two_level_without_final(ssd):
    w = _wl(2, 200, 4, 1, 128, 64, True)
    inp = make_inputs(w, seed=98)
    dev = device_inputs(inp, "bf16")
    g, dtt = _cumsum(ssd, dev, w)
    states, _ = _two_level(ssd, dev, w, g, dtt, with_final=False)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=64, want_y=False)
    assert_close(_np(states), ref["states"], "bf16", "states (no final)")


def _chunk_contributions(inp, T):
    """P_c: the oracle's final state over chunk c alone from a zero state."""
    L = inp["x"].shape[1]
    out = []
    for t0 in range(0, L, T):
        sl = {k: (None if v is None or k in ("A", "D", "init_state") else v[:, t0:t0 + T])
              for k, v in inp.items()}
        r = oracle.forward(sl["x"], sl["dt"], inp["A"], sl["B"], sl["C"], inp["D"], None,
                           chunk_size=T, want_y=False, want_states=False)
        out.append(r["final"])
    return np.stack(out, axis=2)           # [b, H, nc, P, N]


@pytest.mark.parametrize("T,N", [(64, 128), (256, 64)])
def test_chunk_state_alone(ssd, T, N):
    w = _wl(2, 2 * T + 17, 3, 1, N, T, False)
    inp = make_inputs(w, seed=99)
    dev = device_inputs(inp, "bf16")
    g, dtt = _cumsum(ssd, dev, w)
    b, H, P, nc = w.batch, w.nheads, w.headdim, w.nchunks
    states = torch.full((b, H, nc, P, N), float("nan"), device=DEV)
    fin = torch.full((b, H, P, N), float("nan"), device=DEV)
    ssd.ssd_chunk_state(dev["x"], dev["B"], dtt, g, states, fin, T)
    torch.cuda.synchronize()
    pc = _chunk_contributions(inp, T)
    assert torch.isnan(states[:, :, 0]).all()          # slot 0 is not touched
    assert_close(_np(states[:, :, 1:]), pc[:, :, :-1], "bf16", "P_c")
    assert_close(_np(fin), pc[:, :, -1], "bf16", "P_last")


def test_state_passing_alone(ssd):
    w = _wl(2, 300, 4, 2, 128, 64, True)
    inp = make_inputs(w, seed=100)
    dev = device_inputs(inp, "bf16")
    g, _ = _cumsum(ssd, dev, w)
    pc = _chunk_contributions(inp, 64)
    states = torch.from_numpy(np.ascontiguousarray(
        np.concatenate([np.zeros_like(pc[:, :, :1]), pc[:, :, :-1]], axis=2),
        dtype=np.float32)).to(DEV)
    fin = torch.from_numpy(np.ascontiguousarray(pc[:, :, -1], dtype=np.float32)).to(DEV)
    ssd.ssd_state_passing(g, dev["init_state"], states, fin, 64)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=64, want_y=False)
    assert_close(_np(states), ref["states"], "fp32", "states")
    assert_close(_np(fin), ref["final"], "fp32", "final")


def test_two_level_long_full(ssd):
    """The long workload (65536 tokens, 512 chunks): every element of the
    states and the final state."""
    w = WORKLOADS["long_bf16"]
    inp = make_inputs(w)
    log(f"[two-level] full size {w.name}")
    dev = device_inputs(inp, "bf16")
    g, dtt = _cumsum(ssd, dev, w)
    states, fin = _two_level(ssd, dev, w, g, dtt)
    npairs = w.batch * w.nheads
    sp = states.reshape(npairs, w.nchunks, 64, w.dstate)
    fp = fin.reshape(npairs, 64, w.dstate)

    def ref(p0, p1):
        return oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                              inp["init_state"], chunk_size=w.chunk_size,
                              pairs=list(range(p0, p1)), want_y=False)

    def got(p0, p1):
        return {"states": _np(sp[p0:p1]), "final": _np(fp[p0:p1])}

    compare_all_pairs(ref, got, npairs, 16, "bf16", ("states", "final"))


@pytest.mark.parametrize("L,T", [(16384, 128), (8192, 64)])
def test_fwd_pass_state_init_aliases_final(ssd, L, T):
    """init_state and final_state as one buffer (a sequence continued in
    place) give the same states and final state as separate buffers: 128
    chunks of 128 tokens on 4 heads take the two-level form, 128 chunks of
    64 the one-pass kernel."""
    w = _wl(1, L, 4, 1, 128, T, True)
    inp = make_inputs(w, seed=101)
    log(f"[alias] {w}")
    dev = device_inputs(inp, "bf16")
    g, dtt = _cumsum(ssd, dev, w)
    b, H, nc = w.batch, w.nheads, w.nchunks
    s1 = torch.empty(b, H, nc, 64, 128, device=DEV)
    f1 = torch.empty(b, H, 64, 128, device=DEV)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dtt, g, dev["init_state"], s1, f1, T)
    s2 = torch.empty_like(s1)
    both = dev["init_state"].clone()
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dtt, g, both, s2, both, T)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2)
    assert torch.equal(f1, both)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T, want_y=False)
    assert_close(_np(s2), ref["states"], "bf16", "states (aliased)")
    assert_close(_np(both), ref["final"], "bf16", "final (aliased)")
