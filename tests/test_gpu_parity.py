"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Small cases compare every output element; they span several tiles, a ragged
last chunk, grouped B/C and both input types.  The named workloads run at
full size, in the same launch configuration the benchmark times, and compare
every element too, in batches of (batch, head) pairs that the oracle
computes one batch at a time.
"""
import numpy as np
import pytest
import torch

import oracle
from closed_forms import rel_err
from gpu_util import (assert_close, compare_all_pairs, device_inputs, g_tolerance, log,
                      pairs_per_batch)
from ssd_workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _wl(name, dtype, b, L, H, G, N, T, init, dt_shift=-2.0, a=(0.0, 1.5)):
    return Workload(name, b, L, H, 64, N, G, T, dtype, dt_shift, a[0], a[1],
                    0.1 if init else None)


SMALL = [
    _wl("bf16_T64_N128_ragged_grouped", "bf16", 2, 300, 4, 2, 128, 64, True),
    _wl("bf16_T256_N64_ragged", "bf16", 1, 700, 3, 1, 64, 256, False),
    _wl("bf16_T128_N128_init", "bf16", 2, 333, 2, 1, 128, 128, True),
    _wl("bf16_T256_N128_two_chunks", "bf16", 1, 512, 2, 1, 128, 256, True),
    _wl("fp32_T64_N64_grouped", "fp32", 2, 200, 6, 3, 64, 64, True, -1.0, (-1.0, 2.0)),
    _wl("fp32_T128_N128", "fp32", 1, 520, 2, 2, 128, 128, False),
    _wl("fp32_T256_N128_ragged", "fp32", 1, 600, 2, 1, 128, 256, True),
    _wl("fp32_T64_N128_wide_batch", "fp32", 5, 130, 3, 1, 128, 64, False),
    _wl("bf16_T64_N64_shorter_than_chunk", "bf16", 3, 37, 2, 1, 64, 64, False),
    _wl("bf16_T64_N64_grouped_init", "bf16", 2, 450, 6, 3, 64, 64, True),
    # shapes that select each bf16 state-pass tile (heads x columns per
    # workgroup) in the stage-2 call; with an even group size ssd_forward
    # takes the bf16 fused pass on them
    _wl("bf16_T64_N128_3head_tiles", "bf16", 22, 130, 6, 1, 128, 64, True),
    _wl("bf16_T64_N128_half_head_tiles_ragged_init", "bf16", 16, 200, 6, 1, 128, 64, True),
    _wl("bf16_T128_N128_half_head_tiles_grouped", "bf16", 4, 260, 30, 3, 128, 128, False),
    _wl("bf16_T128_N128_whole_head_tiles_grouped", "bf16", 16, 300, 10, 2, 128, 128, False),
    _wl("bf16_T64_N128_whole_head_tiles_ragged_init", "bf16", 2, 130, 80, 1, 128, 64, True),
    _wl("bf16_T64_N128_4head_tiles_grouped", "bf16", 4, 100, 32, 4, 128, 64, True),
    _wl("bf16_T256_N128_2head_tiles_ragged", "bf16", 8, 300, 8, 1, 128, 256, True),
    _wl("bf16_T64_N128_4head_tiles", "bf16", 16, 100, 8, 1, 128, 64, False),
    _wl("bf16_T128_N128_1head_tiles_group_per_head", "bf16", 4, 150, 8, 8, 128, 128, True),
    _wl("bf16_T128_N128_single_token", "bf16", 1, 1, 1, 1, 128, 128, True),
    _wl("fp32_T256_N64_single_token", "fp32", 2, 1, 2, 2, 64, 256, True),
    # decay extremes: A dt from about -0.5 to -70 per token (most exponents
    # underflow within a few tokens), and from -2e-6 to -1e-3 per token (the
    # state keeps nearly the whole sequence)
    _wl("bf16_T128_N128_strong_decay", "bf16", 2, 300, 4, 2, 128, 128, True, 1.0, (2.0, 3.0)),
    _wl("bf16_T256_N64_weak_decay_init", "bf16", 1, 900, 3, 1, 64, 256, True, -4.0, (-6.0, -5.0)),
    _wl("fp32_T64_N128_strong_decay", "fp32", 2, 200, 3, 3, 128, 64, False, 1.0, (2.0, 3.0)),
    # fp32 shapes with enough (batch, head) pairs for the state-pass kernel
    # whose workgroups share B among 3 or 2 heads of a group
    _wl("fp32_T64_N64_3head_shared_B_ragged_init", "fp32", 128, 70, 6, 2, 64, 64, True,
        -1.0, (-1.0, 2.0)),
    _wl("fp32_T128_N128_2head_shared_B", "fp32", 128, 300, 4, 2, 128, 128, False),
    _wl("fp32_T256_N128_3head_shared_B_ragged", "fp32", 86, 260, 9, 3, 128, 256, True),
    _wl("fp32_T64_N64_3head_shared_B_one_chunk", "fp32", 64, 64, 12, 2, 64, 64, False,
        -1.0, (-1.0, 2.0)),
    # fp32, 64-token chunks, N 64, at least one (batch, head pair) per compute
    # unit: ssd_forward runs stages 2 and 3 as one fused pass (two heads per
    # workgroup where the group size is even, one where it is odd)
    _wl("fp32_T64_N64_fused_pairs_ragged_init", "fp32", 48, 300, 12, 2, 64, 64, True,
        -1.0, (-1.0, 2.0)),
    _wl("fp32_T64_N64_fused_single_heads", "fp32", 32, 200, 9, 3, 64, 64, False,
        -1.0, (-1.0, 2.0)),
    _wl("fp32_T64_N64_fused_two_pairs_per_workgroup_init", "fp32", 128, 130, 8, 1, 64, 64, True),
    _wl("fp32_T64_N64_fused_weak_decay_short", "fp32", 96, 40, 6, 3, 64, 64, True,
        -4.0, (-6.0, -5.0)),
    # groups of three heads (odd group size: the stage-2 call keeps the
    # fp32-instruction kernel, ssd_forward the single-head fused pass),
    # ragged, with init
    _wl("fp32_T64_N64_head_triples_ragged_init", "fp32", 96, 200, 9, 3, 64, 64, True,
        -1.0, (-1.0, 2.0)),
]


def _run_forward(ssd, dev, T, y_dtype=torch.float32):
    y, states, final = ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"],
                                   dev["C"], dev["D"], dev["init_state"],
                                   chunk_size=T, y_dtype=y_dtype)
    torch.cuda.synchronize()
    return y, states, final


def _np(t):
    return t.detach().float().cpu().numpy()


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
def test_small_end_to_end(ssd, w):
    log(f"[parity] {w.name}: b={w.batch} L={w.seqlen} H={w.nheads} "
        f"G={w.ngroups} N={w.dstate} T={w.chunk_size} {w.dtype}")
    inp = make_inputs(w, seed=11)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    dev = device_inputs(inp, w.dtype)
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    assert_close(_np(states), ref["states"], w.dtype, "states")
    assert_close(_np(final), ref["final"], w.dtype, "final")
    assert_close(_np(y), ref["y"], w.dtype, "y")


# the stage calls on the first eight shapes and on every bf16 shape with
# N = 128 (ssd_forward runs those as the fused pass, so the state-pass tiles
# they were chosen to select are reached through the stage calls here)
STAGE_CASES = SMALL[:8] + [w for w in SMALL[8:] if w.dtype == "bf16" and w.dstate == 128]
# fp32 shapes with 64-token chunks and N = 64: with an even group size and
# at least one (batch, head pair) per compute unit the stage-2 call runs the
# head-pair state kernel on them (ragged and single partial chunks, init,
# several pairs per workgroup; strong decay is compared path to path in
# test_fused_forward_matches_stage_calls), with an odd one the
# fp32-instruction kernel
STAGE_CASES += [w for w in SMALL if w.name in (
    "fp32_T64_N64_3head_shared_B_one_chunk", "fp32_T64_N64_fused_pairs_ragged_init",
    "fp32_T64_N64_fused_two_pairs_per_workgroup_init", "fp32_T64_N64_fused_weak_decay_short",
    "fp32_T64_N64_head_triples_ragged_init")]


@pytest.mark.parametrize("w", STAGE_CASES, ids=lambda w: w.name)
def test_small_stages(ssd, w):
    log(f"[stages] {w.name}")
    T = w.chunk_size
    inp = make_inputs(w, seed=12)
    dev = device_inputs(inp, w.dtype)
    b, L, H = w.batch, w.seqlen, w.nheads
    nc = w.nchunks
    # stage 1 against the oracle's cumsum, within the fp32 rounding bound;
    # its transposed dt copy is exact
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    torch.cuda.synchronize()
    g_ref = oracle.chunk_cumsum(inp["dt"], inp["A"], T)
    err = np.abs(_np(g) - g_ref)
    assert np.all(err <= g_tolerance(g_ref, T)), float(err.max())
    assert np.array_equal(_np(dt_t), inp["dt"].transpose(0, 2, 1))
    # stage 2 (fed the GPU g) against the recurrence's chunk states
    states = torch.empty(b, H, nc, 64, w.dstate, device=DEV)
    final = torch.empty(b, H, 64, w.dstate, device=DEV)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"],
                           states, final, T)
    torch.cuda.synchronize()
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=T)
    assert_close(_np(states), ref["states"], w.dtype, "stage-2 states")
    assert_close(_np(final), ref["final"], w.dtype, "stage-2 final")
    # stage 3 fed the oracle's states (rounded to fp32), against the oracle's
    # chunk outputs from those same fp32 states
    st32 = ref["states"].astype(np.float32)
    y = torch.empty(tuple(dev["x"].shape), dtype=torch.float32, device=DEV)
    ssd.ssd_compute_out(dev["x"], dev["B"], dev["C"], dt_t, g,
                        torch.from_numpy(st32).to(DEV), dev["D"], y, T)
    torch.cuda.synchronize()
    y_ref = oracle.chunk_out(inp["x"], inp["dt"], inp["A"], inp["B"],
                             inp["C"], inp["D"], st32, chunk_size=T)
    assert_close(_np(y), y_ref, w.dtype, "stage-3 y")


def test_cumsum_exact_inputs(ssd):
    # A = -1 and dt powers of two: products and partial sums are exact in
    # fp32, so g differs from the oracle only by the final log2(e) scaling.
    b, L, H, T = 2, 300, 5, 64
    rng = np.random.default_rng(3)
    dt = (2.0 ** rng.integers(-6, 2, size=(b, L, H))).astype(np.float32)
    A = -np.ones(H, np.float32)
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(torch.from_numpy(dt).to(DEV), torch.from_numpy(A).to(DEV), g, dt_t, T)
    torch.cuda.synchronize()
    g_ref = oracle.chunk_cumsum(dt, A, T)
    err = np.abs(_np(g) - g_ref)
    assert np.all(err <= 2.0 ** -22 * np.abs(g_ref)), float((err / np.abs(g_ref)).max())


# ------------------------------------------------------ named full workloads
NAMED = ["tiny_fp32", "small_bf16", "large_bf16", "wide_fp32", "long_bf16"]


@pytest.mark.parametrize("name", NAMED)
def test_named_workload_full_size(ssd, name):
    """Every element of y, states and final at the workload's full size, in
    the launch configuration the benchmark times, against the oracle (pairs
    of (batch, head) in batches to bound host memory)."""
    w = WORKLOADS[name]
    log(f"[full] {name}: b={w.batch} L={w.seqlen} H={w.nheads} N={w.dstate} "
        f"G={w.ngroups} T={w.chunk_size} {w.dtype}")
    inp = make_inputs(w)
    dev = device_inputs(inp, w.dtype)
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    b, L, H, P, N, nc = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.nchunks
    # pair-major views of the device outputs: pair = b * H + h
    yp = y.permute(0, 2, 1, 3).reshape(b * H, L, P)
    sp = states.reshape(b * H, nc, P, N)
    fp = final.reshape(b * H, P, N)

    def ref(p0, p1):
        return oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                              inp["D"], inp["init_state"], chunk_size=w.chunk_size,
                              pairs=list(range(p0, p1)))

    def got(p0, p1):
        return {"y": _np(yp[p0:p1]), "states": _np(sp[p0:p1]), "final": _np(fp[p0:p1])}

    compare_all_pairs(ref, got, b * H, pairs_per_batch(w), w.dtype,
                      ("states", "final", "y"))
    if inp["init_state"] is None:
        assert bool((states[:, :, 0] == 0).all())
    else:
        assert torch.equal(states[:, :, 0], dev["init_state"])


# whole run against two halves: the bf16 fused pass cuts each chain into
# runs whose starting states come from the run pass, and the two calls cut
# it at other chunks, so the two sum the same fp32 terms in other orders
# (measured below 1e-5 relative)
SPLIT_TOL = 1e-4


def test_long_sequence_split_in_halves_matches_whole(ssd):
    """The final state of the 65536-token sequence equals that of its two
    halves run back to back (the second from the first's final state), and
    so do y and every chunk's state, to fp32 summation order."""
    w = WORKLOADS["long_bf16"]
    log(f"[split] {w.name}: whole vs two halves of {w.seqlen // 2}")
    inp = make_inputs(w)
    dev = device_inputs(inp, w.dtype)
    T = w.chunk_size
    y, states, final = _run_forward(ssd, dev, T)
    half = w.seqlen // 2
    first = {k: (v[:, :half].contiguous() if k in ("x", "B", "C", "dt") else v)
             for k, v in dev.items()}
    y1, s1, f1 = _run_forward(ssd, first, T)
    second = {k: (v[:, half:].contiguous() if k in ("x", "B", "C", "dt") else v)
              for k, v in dev.items()}
    second["init_state"] = f1
    y2, s2, f2 = _run_forward(ssd, second, T)
    assert torch.equal(s2[:, :, 0], f1)
    for what, a, b_ in (("final", f2, final), ("states", torch.cat([s1, s2], 2), states),
                        ("y", torch.cat([y1, y2], 1), y)):
        e = rel_err(_np(a), _np(b_))
        log(f"  {what}: halves vs whole rel(RMS-floored)={e:.3e}")
        assert e <= SPLIT_TOL, (what, e)


# ----------------------------------------------------------- special cases
def _small_inputs(seed=21, dtype="bf16", b=2, L=200, H=4, G=2, N=128, T=64,
                  init=True):
    w = _wl("special", dtype, b, L, H, G, N, T, init)
    return w, make_inputs(w, seed=seed)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_dt_passes_state_through_exactly(ssd, dtype):
    w, inp = _small_inputs(dtype=dtype)
    inp["dt"] = np.zeros_like(inp["dt"])
    dev = device_inputs(inp, dtype)
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    init = dev["init_state"]
    for c in range(w.nchunks):
        assert torch.equal(states[:, :, c], init)
    assert torch.equal(final, init)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], dtype, "y = C h0 + D x")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_no_decay_matches_oracle(ssd, dtype):
    w, inp = _small_inputs(dtype=dtype, seed=22)
    inp["A"] = np.zeros_like(inp["A"])
    dev = device_inputs(inp, dtype)
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], dtype, "y")
    assert_close(_np(final), ref["final"], dtype, "final")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_extreme_decay_is_finite_and_matches(ssd, dtype):
    w, inp = _small_inputs(dtype=dtype, seed=23, T=256, L=600)
    inp["A"] = (inp["A"] * 1e4).astype(np.float32)     # a_t << -100
    dev = device_inputs(inp, dtype)
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    assert bool(torch.isfinite(y).all())
    assert bool(torch.isfinite(states).all()) and bool(torch.isfinite(final).all())
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], dtype, "y")
    assert_close(_np(final), ref["final"], dtype, "final")


def test_zero_inputs_give_zero_outputs(ssd):
    w, inp = _small_inputs(seed=24, init=False)
    inp["x"] = np.zeros_like(inp["x"])
    dev = device_inputs(inp, "bf16")
    y, states, final = _run_forward(ssd, dev, w.chunk_size)
    assert bool((y == 0).all()) and bool((states == 0).all())
    assert bool((final == 0).all())


def test_deterministic_and_fully_written(ssd):
    w, inp = _small_inputs(seed=25, L=333)
    dev = device_inputs(inp, "bf16")
    d = ssd.make_dims(dev["x"], dev["B"], w.chunk_size)
    outs = []
    for _ in range(2):
        y = torch.full(tuple(dev["x"].shape), float("nan"), device=DEV)
        st = torch.full((w.batch, w.nheads, w.nchunks, 64, w.dstate),
                        float("nan"), device=DEV)
        fin = torch.full((w.batch, w.nheads, 64, w.dstate), float("nan"), device=DEV)
        ws = torch.full((ssd.workspace_bytes(d) // 4,), float("nan"), device=DEV)
        ssd.ssd_forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"],
                        dev["D"], dev["init_state"], y, st, fin, ws, w.chunk_size)
        torch.cuda.synchronize()
        assert not bool(torch.isnan(y).any())
        assert not bool(torch.isnan(st).any()) and not bool(torch.isnan(fin).any())
        outs.append((y, st, fin))
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)


def test_forward_equals_stage_calls(ssd):
    # N = 64: ssd_forward runs the stage-2 and stage-3 kernels themselves
    w, inp = _small_inputs(seed=26, L=257, T=128, N=64)
    dev = device_inputs(inp, "bf16")
    T = w.chunk_size
    y, states, final = _run_forward(ssd, dev, T)
    b, L, H = w.batch, w.seqlen, w.nheads
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    s2 = torch.empty_like(states)
    f2 = torch.empty_like(final)
    y2 = torch.empty_like(y)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], s2, f2, T)
    ssd.ssd_compute_out(dev["x"], dev["B"], dev["C"], dt_t, g, s2, dev["D"], y2, T)
    torch.cuda.synchronize()
    assert torch.equal(s2, states) and torch.equal(f2, final) and torch.equal(y2, y)


def _fused_case(seed, init=True, dt_shift=-1.0, a=(-1.0, 2.0), H=14, G=7):
    # 40 x 14 heads in groups of 2: 280 (batch, head pair) workgroups
    w = _wl("fused_check", "fp32", 40, 250, H, G, 64, 64, init, dt_shift, a)
    return w, make_inputs(w, seed=seed)


# fused pass against the two-kernel path on the same g: both sum the same
# fp32 products in different orders (measured 2e-6 and below)
FUSED_VS_STAGES_TOL = 2e-5


@pytest.mark.parametrize("regime", ["moderate_decay_pairs", "extreme_decay_single_heads",
                                    "extreme_decay_pairs"])
def test_fused_forward_matches_stage_calls(ssd, regime):
    """The fused pass of ssd_forward and the separate stage-2 and stage-3
    kernels agree to fp32 rounding (they sum in different orders).

    The extreme regime (A dt from about -10 to -26 per token) makes |g| reach
    thousands within a chunk, where fp32 keeps g to an absolute 2^-24 |g|:
    the stage-1 rounding then moves decay factors by about 1e-4 relative on
    either path, which is why this regime is compared path to path, with the
    final state (a sum the last tokens dominate) against the oracle."""
    if regime == "moderate_decay_pairs":
        w, inp = _fused_case(31)
    elif regime == "extreme_decay_single_heads":
        w, inp = _fused_case(34, init=False, dt_shift=1.0, a=(2.0, 3.0), H=9, G=3)
    else:
        # groups of two heads: the stage-2 call runs the head-pair state kernel
        w, inp = _fused_case(37, init=True, dt_shift=1.0, a=(2.0, 3.0))
    log(f"[fused] {regime} {w}")
    dev = device_inputs(inp, "fp32")
    T = w.chunk_size
    y, states, final = _run_forward(ssd, dev, T)
    b, L, H = w.batch, w.seqlen, w.nheads
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    s2 = torch.empty_like(states)
    f2 = torch.empty_like(final)
    y2 = torch.empty_like(y)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], s2, f2, T)
    ssd.ssd_compute_out(dev["x"], dev["B"], dev["C"], dt_t, g, s2, dev["D"], y2, T)
    torch.cuda.synchronize()
    for what, a, b_ in (("states", states, s2), ("final", final, f2), ("y", y, y2)):
        assert bool(torch.isfinite(a).all())
        e = rel_err(_np(a), _np(b_))
        log(f"  {what}: fused vs stages rel(RMS-floored)={e:.3e}")
        assert e <= FUSED_VS_STAGES_TOL, (what, e)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=T, want_y=False)
    assert_close(_np(final), ref["final"], "fp32", "final (fused)")


@pytest.mark.parametrize("case", ["fused_fp32", "fused_bf16_runs", "two_kernel_bf16"])
def test_state_and_out_entry_point(ssd, case):
    """ssd_state_and_out on stage 1's outputs gives exactly what ssd_forward
    gives (same kernels), on shapes that take the fp32 and the bf16 fused
    passes and on one that takes the two stage kernels (there also exactly
    the separate stage-2 and stage-3 calls)."""
    if case == "fused_fp32":
        w, inp = _fused_case(35)
        dtype = "fp32"
    elif case == "fused_bf16_runs":
        w, inp = _small_inputs(seed=37, L=1000, T=128, N=128)
        dtype = "bf16"
    else:
        w, inp = _small_inputs(seed=36, L=257, T=128, N=64)
        dtype = "bf16"
    dev = device_inputs(inp, dtype)
    T = w.chunk_size
    y, states, final = _run_forward(ssd, dev, T)
    b, L, H = w.batch, w.seqlen, w.nheads
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    y2, s2, f2 = torch.empty_like(y), torch.empty_like(states), torch.empty_like(final)
    ssd.ssd_state_and_out(dev["x"], dev["B"], dev["C"], dt_t, g, dev["D"], dev["init_state"],
                          y2, s2, f2, T)
    torch.cuda.synchronize()
    assert torch.equal(y2, y) and torch.equal(s2, states) and torch.equal(f2, final)
    if case == "two_kernel_bf16":
        s3, f3, y3 = torch.empty_like(states), torch.empty_like(final), torch.empty_like(y)
        ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], s3, f3, T)
        ssd.ssd_compute_out(dev["x"], dev["B"], dev["C"], dt_t, g, s3, dev["D"], y3, T)
        torch.cuda.synchronize()
        assert torch.equal(s3, s2) and torch.equal(f3, f2) and torch.equal(y3, y2)


def test_fused_forward_init_aliases_final(ssd):
    """ssd_forward on the fused path with init_state and final_state as one
    buffer gives what separate buffers give."""
    w, inp = _fused_case(32)
    dev = device_inputs(inp, "fp32")
    T = w.chunk_size
    b, L, H, nc = w.batch, w.seqlen, w.nheads, w.nchunks
    ws = torch.empty(ssd.workspace_bytes(ssd.make_dims(dev["x"], dev["B"], T)),
                     dtype=torch.uint8, device=DEV)
    outs = []
    for alias in (False, True):
        y = torch.empty_like(dev["x"])
        st = torch.empty(b, H, nc, 64, 64, device=DEV)
        init = dev["init_state"].clone()
        fin = init if alias else torch.empty_like(init)
        ssd.ssd_forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], init,
                        y, st, fin, ws, T)
        torch.cuda.synchronize()
        outs.append((y, st, fin))
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T)
    assert_close(_np(outs[1][2]), ref["final"], "fp32", "final (aliased)")


def test_state_pass_init_aliases_final(ssd):
    """ssd_fwd_pass_state with init_state and final_state as one buffer (a
    sequence continued in place) gives what separate buffers give, on the
    head-pair fp32 state kernel (280 pairs, 4 chunks, ragged)."""
    w, inp = _fused_case(36)
    dev = device_inputs(inp, "fp32")
    T = w.chunk_size
    b, L, H, nc = w.batch, w.seqlen, w.nheads, w.nchunks
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    outs = []
    for alias in (False, True):
        st = torch.full((b, H, nc, 64, 64), float("nan"), device=DEV)
        init = dev["init_state"].clone()
        fin = init if alias else torch.empty_like(init)
        ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, init, st, fin, T)
        torch.cuda.synchronize()
        outs.append((st, fin))
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["init_state"], chunk_size=T)
    assert_close(_np(outs[1][0]), ref["states"], "fp32", "stage-2 states (aliased)")
    assert_close(_np(outs[1][1]), ref["final"], "fp32", "stage-2 final (aliased)")


def test_wide_state_pass_full_size(ssd):
    """The stage-2 call alone at the wide fp32 layer's full size (64 x 1024
    tokens, 48 heads in 8 groups: the head-pair state kernel), every state
    and final element against the oracle."""
    w = WORKLOADS["wide_fp32"]
    log(f"[full stage 2] {w}")
    inp = make_inputs(w)
    dev = device_inputs(inp, w.dtype)
    T = w.chunk_size
    b, L, H, P, N, nc = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.nchunks
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    states = torch.full((b, H, nc, P, N), float("nan"), device=DEV)
    final = torch.full((b, H, P, N), float("nan"), device=DEV)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], states, final, T)
    torch.cuda.synchronize()
    sp = states.reshape(b * H, nc, P, N)
    fp = final.reshape(b * H, P, N)

    def ref(p0, p1):
        r = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                           inp["init_state"], chunk_size=T, pairs=list(range(p0, p1)),
                           want_y=False)
        return {"states": r["states"], "final": r["final"]}

    def got(p0, p1):
        return {"states": _np(sp[p0:p1]), "final": _np(fp[p0:p1])}

    compare_all_pairs(ref, got, b * H, pairs_per_batch(w), w.dtype, ("states", "final"),
                      label="stage 2: ")


def test_fused_forward_bf16_output(ssd):
    w, inp = _fused_case(33, init=False)
    dev = device_inputs(inp, "fp32")
    y, _, _ = _run_forward(ssd, dev, w.chunk_size, y_dtype=torch.bfloat16)
    assert y.dtype == torch.bfloat16
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], "fp32", "bf16 y (fused)", y_bf16=True)


# ------------------------------------------------- bf16 fused pass (runs)
# Shapes that give the bf16 fused pass each plan on a 256-CU device (pairs =
# batch x heads / 2; R = ceil(pairs x chunks / CUs) chunk steps per CU, a
# lead run of R0 = chunks - (nr - 1) R and nr - 1 runs of R):
#  * one run per chain, more pairs than workgroups (a workgroup takes several
#    (b, pair) items in turn): 32 x 24 heads = 384 pairs;
#  * 16 pairs, 40 chunks: runs of 3 after a lead run of 1, ragged, init;
#  * 100 pairs, 6 chunks: two runs of 3, groups of 2 heads;
#  * lead runs of 2 (1) chunks, three (two) of them to a workgroup, as at the
#    small and large layers;
#  * 256-token chunks walked as four 64-token blocks, ragged, one chunk a run;
#  * 128-token chunks, groups of 4 heads, init.
FUSED_BF16 = [
    _wl("persistent_pairs_T64", "bf16", 32, 200, 24, 1, 128, 64, False),
    _wl("runs_of_3_lead_1_T64_ragged_init", "bf16", 1, 2553, 32, 1, 128, 64, True),
    _wl("two_runs_T64_grouped", "bf16", 1, 380, 200, 2, 128, 64, True),
    # lead runs shorter than the others, three (two) to a workgroup
    _wl("lead_runs_3_per_wg_T64_ragged_init", "bf16", 2, 2000, 48, 1, 128, 64, True),
    _wl("lead_runs_2_per_wg_T256_init", "bf16", 1, 4000, 88, 1, 128, 256, True),
    _wl("blocks_in_T256_ragged_init", "bf16", 1, 1380, 4, 1, 128, 256, True),
    _wl("T128_groups_of_4_init", "bf16", 3, 1000, 8, 2, 128, 128, True),
]

# bf16 fused pass against the two stage kernels on the same g and dt_t:
# both sum fp32 terms of the same bf16 operands, the computed operands split
# hi + lo on both (measured below 1e-4)
FUSED_BF16_VS_STAGES_TOL = 1e-3


@pytest.mark.parametrize("w", FUSED_BF16, ids=lambda w: w.name)
def test_fused_bf16_forward(ssd, w):
    """ssd_forward on the bf16 fused pass against the oracle (every
    element) and against the separate stage-2 and stage-3 kernels."""
    log(f"[fused bf16] {w}")
    inp = make_inputs(w, seed=41)
    dev = device_inputs(inp, "bf16")
    T = w.chunk_size
    y, states, final = _run_forward(ssd, dev, T)
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=T)
    assert_close(_np(states), ref["states"], "bf16", "states")
    assert_close(_np(final), ref["final"], "bf16", "final")
    assert_close(_np(y), ref["y"], "bf16", "y")
    b, L, H = w.batch, w.seqlen, w.nheads
    g = torch.empty(b, H, L, device=DEV)
    dt_t = torch.empty(b, H, L, device=DEV)
    s2, f2, y2 = torch.empty_like(states), torch.empty_like(final), torch.empty_like(y)
    ssd.ssd_chunk_cumsum(dev["dt"], dev["A"], g, dt_t, T)
    ssd.ssd_fwd_pass_state(dev["x"], dev["B"], dt_t, g, dev["init_state"], s2, f2, T)
    ssd.ssd_compute_out(dev["x"], dev["B"], dev["C"], dt_t, g, s2, dev["D"], y2, T)
    torch.cuda.synchronize()
    for what, a, b_ in (("states", states, s2), ("final", final, f2), ("y", y, y2)):
        e = rel_err(_np(a), _np(b_))
        log(f"  {what}: fused vs stages rel(RMS-floored)={e:.3e}")
        assert e <= FUSED_BF16_VS_STAGES_TOL, (what, e)


@pytest.mark.parametrize("runs", ["one_run", "several_runs"])
def test_fused_bf16_init_aliases_final(ssd, runs):
    """init_state and final_state as one buffer on the bf16 fused pass,
    with one run per chain (the fused kernel reads init and writes final)
    and with several (the run passing reads init, the fused kernel the
    states)."""
    if runs == "one_run":
        w = FUSED_BF16[0].with_(init_std=0.1)
    else:
        w = FUSED_BF16[1]
    inp = make_inputs(w, seed=42)
    dev = device_inputs(inp, "bf16")
    T = w.chunk_size
    b, L, H, nc = w.batch, w.seqlen, w.nheads, w.nchunks
    ws = torch.empty(ssd.workspace_bytes(ssd.make_dims(dev["x"], dev["B"], T)),
                     dtype=torch.uint8, device=DEV)
    outs = []
    for alias in (False, True):
        y = torch.empty(b, L, H, 64, device=DEV)
        st = torch.empty(b, H, nc, 64, 128, device=DEV)
        init = dev["init_state"].clone()
        fin = init if alias else torch.empty_like(init)
        ssd.ssd_forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"], init,
                        y, st, fin, ws, T)
        torch.cuda.synchronize()
        outs.append((y, st, fin))
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a, b_)


def test_fused_bf16_output(ssd):
    w = FUSED_BF16[3]
    inp = make_inputs(w, seed=43)
    dev = device_inputs(inp, "bf16")
    y, _, _ = _run_forward(ssd, dev, w.chunk_size, y_dtype=torch.bfloat16)
    assert y.dtype == torch.bfloat16
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], "bf16", "bf16 y (fused)", y_bf16=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bf16_output(ssd, dtype):
    w, inp = _small_inputs(seed=27, dtype=dtype)
    dev = device_inputs(inp, dtype)
    y, _, _ = _run_forward(ssd, dev, w.chunk_size, y_dtype=torch.bfloat16)
    assert y.dtype == torch.bfloat16
    ref = oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                         inp["D"], inp["init_state"], chunk_size=w.chunk_size)
    assert_close(_np(y), ref["y"], dtype, "bf16 y", y_bf16=True)


def test_binding_rejects_bad_arguments(ssd):
    w, inp = _small_inputs(seed=28)
    dev = device_inputs(inp, "bf16")
    with pytest.raises(ValueError):     # wrong dt shape
        ssd.forward(dev["x"], dev["dt"][:, :-1].contiguous(), dev["A"], dev["B"],
                    dev["C"], dev["D"], chunk_size=64)
    with pytest.raises(TypeError):      # B dtype differs from x
        ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"].float(), dev["C"],
                    dev["D"], chunk_size=64)
    dt_off = torch.empty(dev["dt"].numel() + 1, device=DEV)[1:].view(dev["dt"].shape)
    dt_off.copy_(dev["dt"])
    with pytest.raises(ValueError):     # contiguous, but 4 bytes past a 16-byte boundary
        ssd.forward(dev["x"], dt_off, dev["A"], dev["B"], dev["C"], dev["D"], chunk_size=64)
    with pytest.raises(ssd.SsdError) as e:   # chunk size not built
        ssd.forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"],
                    dev["D"], chunk_size=32)
    assert e.value.status == ssd.SSD_ERR_UNSUPPORTED
