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


# ---- fp32 layers with many (batch, head) chains: 64-token chunks, N = 64,
# at least 512 chains, so ssd_forward runs the fused pass and the stage-2
# call the head-pair state kernel (where the group size is even) or the
# fp32-instruction one; both against the oracle

def _draw_many(n=8, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.choice([2, 4, 6, 8, 12]))
        G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
        b = -(-512 // H) + int(rng.integers(0, 40))
        L = int(rng.integers(1, 301))
        out.append((i, b, L, H, G, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("case", _draw_many(), ids=lambda c: "m%02d_b%d_L%d_H%d_G%d%s" % (
    c[0], c[1], c[2], c[3], c[4], "_init" if c[5] else ""))
def test_random_many_chains_fp32(ssd, case):
    i, b, L, H, G, init = case
    w = Workload("many", b, L, H, 64, 64, G, 64, "fp32", -1.0, -1.0, 2.0, 0.1 if init else None)
    log(f"[random many] {case}")
    inp = make_inputs(w, seed=700 + i)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=64)
    dev = device_inputs(inp, "fp32")
    y, states, final = ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"],
                                   dev["D"], dev["init_state"], chunk_size=64)
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, 64)
    s2 = torch.full_like(states, float("nan"))
    f2 = torch.full_like(final, float("nan"))
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], s2, f2, 64)
    torch.cuda.synchronize()
    assert_close(_np(states), ref["states"], "fp32", "states")
    assert_close(_np(final), ref["final"], "fp32", "final")
    assert_close(_np(y), ref["y"], "fp32", "y")
    assert_close(_np(s2), ref["states"], "fp32", "stage-2 states")
    assert_close(_np(f2), ref["final"], "fp32", "stage-2 final")


# ---- the other entry points, drawn the same way

def _draw_conv(n=16, seed=2025):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 4)), int(rng.integers(1, 40)), int(rng.integers(1, 3000)),
             int(rng.integers(1, 5)), str(rng.choice(["bf16", "fp32"])),
             str(rng.choice(["bf16", "fp32"])), bool(rng.integers(0, 2))) for i in range(n)]


@pytest.mark.parametrize("case", _draw_conv(), ids=lambda c: "c%02d_b%d_d%d_L%d_W%d_%s_to_%s%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "" if c[7] else "_nobias"))
def test_random_conv(ssd, case):
    from ssd_workloads import ConvWorkload, make_conv_inputs
    from test_gpu_conv import _check, _run
    i, b, dim, L, W, xdt, odt, bias = case
    c = ConvWorkload("conv_random", b, dim, L, W, xdt, bias)
    inp = make_conv_inputs(c, seed=600 + i)
    log(f"[random conv] {case}")
    _check(_run(ssd, inp, xdt, odt), inp, odt, "conv out")


def _draw_gdn(n=8, seed=2026):
    rng = np.random.default_rng(seed)
    return [(i, int(rng.integers(1, 3)), int(rng.integers(1, 400)), int(rng.integers(1, 5)),
             int(rng.choice([64, 128])), int(rng.choice([64, 128])),
             float(rng.choice([0.0, 0.2]))) for i in range(n)]


@pytest.mark.parametrize("case", _draw_gdn(), ids=lambda c: "g%02d_b%d_L%d_H%d_K%d_V%d%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], "_init" if c[6] else ""))
def test_random_gdn_chain(ssd, case):
    """chunk_fwd_h with fp32 v_new, then chunk_fwd_o fed its output, against
    the oracle's chain at the bf16 tolerance of the Gated DeltaNet suite."""
    from ssd_workloads import GdnWorkload, make_gdn_inputs
    from test_gpu_gdn import _dev, _run_h
    i, b, L, H, K, V, init = case
    c = GdnWorkload("gdn_random", b, L, H, K, V, "bf16", init if init else None)
    inp = make_gdn_inputs(c, seed=700 + i)
    log(f"[random gdn] {case}")
    h, vn, fin = _run_h(ssd, c, inp)
    ref = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    assert_close(_np(h), ref["h"], "bf16", "h")
    assert_close(_np(vn), ref["v_new"], "bf16", "v_new")
    assert_close(_np(fin), ref["final"], "bf16", "final")
    q = _dev(inp, "q")
    # chunk_fwd_o takes a bf16 v_new: feed it the oracle's, rounded, and the
    # oracle's states, so only the output stage is under test here
    vn_b = torch.from_numpy(np.ascontiguousarray(ref["v_new"], np.float32)).to(DEV, torch.bfloat16)
    hs = torch.from_numpy(np.ascontiguousarray(ref["h"], np.float32)).to(DEV)
    o = torch.empty(b, L, H, V, device=DEV)
    ssd.ssd_gdn_chunk_fwd_o(q, _dev(inp, "k"), vn_b, hs, _dev(inp, "g", torch.float32), o,
                            scale=K ** -0.5)
    torch.cuda.synchronize()
    o_ref = oracle.gdn_chunk_fwd_o(inp["q"], inp["k"], _np(vn_b).astype(np.float64),
                                   ref["h"].astype(np.float32).astype(np.float64), inp["g"],
                                   scale=K ** -0.5)
    assert_close(_np(o), o_ref, "bf16", "o")


def _draw_decode(n=8, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        H = int(rng.integers(1, 13))
        G = int(rng.choice([g for g in range(1, H + 1) if H % g == 0]))
        out.append((i, int(rng.integers(1, 9)), H, G, int(rng.choice([64, 128])),
                    str(rng.choice(["bf16", "fp32"]))))
    return out


@pytest.mark.parametrize("case", _draw_decode(), ids=lambda c: "d%02d_b%d_H%d_G%d_N%d_%s" % c)
def test_random_decode(ssd, case):
    """Three decode steps from a random state against the oracle's forward
    over the same three tokens with that state as its initial state."""
    i, b, H, G, N, dtype = case
    L = 3
    w = Workload("decode_random", b, L, H, 64, N, G, 64, dtype, -2.0, 0.0, 1.5, 0.5)
    inp = make_inputs(w, seed=800 + i)
    log(f"[random decode] {case}")
    dev = device_inputs(inp, dtype)
    state = dev["init_state"].clone()
    ys = []
    for t in range(L):
        # fresh copies: a token's slice can be contiguous but not 16-byte
        # aligned (dt of one sequence is 4 * H bytes), which the ABI refuses
        y = torch.empty(b, H, 64, device=DEV)
        ssd.ssd_decode_step(dev["x"][:, t].clone(), dev["dt"][:, t].clone(),
                            dev["A"], dev["B"][:, t].clone(), dev["C"][:, t].clone(),
                            dev["D"], state, y)
        ys.append(y)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=64)
    assert_close(np.stack([_np(y) for y in ys], axis=1), ref["y"], "fp32", "decode y")
    assert_close(_np(state), ref["final"], "fp32", "decode state")
