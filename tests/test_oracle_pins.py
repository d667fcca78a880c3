"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test checks the oracle against a closed form, a hand-computed example,
a special case that reduces to a textbook operation, or an invariant the
pages state.  Together they are chosen so that a dropped term, a wrong sign,
an off-by-one in the state the output reads, a transposed state or a
mis-sampled chunk state fails at least one of them.
"""
import json
import os

import numpy as np
import pytest

import oracle
from closed_forms import (chunked_form, masked_matmul_form, rel_err,
                          unrolled_form)
from ssd_workloads import WORKLOADS, make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "hand_recurrence.json")


def _rand_case(seed, b=2, L=37, H=4, G=2, P=3, N=5, T=8, zero_init=False,
               a_scale=1.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, L, H, P)).astype(np.float32)
    B = rng.standard_normal((b, L, G, N)).astype(np.float32)
    C = rng.standard_normal((b, L, G, N)).astype(np.float32)
    dt = np.logaddexp(0, rng.standard_normal((b, L, H)) - 1).astype(np.float32)
    A = (-np.exp(rng.uniform(-1, 1, H)) * a_scale).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    init = (None if zero_init else
            rng.standard_normal((b, H, P, N)).astype(np.float32))
    return x, dt, A, B, C, D, init, T


def _run(x, dt, A, B, C, D, init, T, **kw):
    return oracle.forward(x, dt, A, B, C, D, init, chunk_size=T, **kw)


# --------------------------------------------------------------- hand values
@pytest.mark.parametrize("case", json.load(open(GOLDEN))["cases"],
                         ids=lambda c: c["name"])
def test_hand_computed_examples(case):
    d = case["dims"]
    b, L, H, P, N, G, T = (d["batch"], d["seqlen"], d["nheads"], d["headdim"],
                           d["dstate"], d["ngroups"], d["chunk_size"])
    arr = lambda k, shp: np.array(case[k], np.float32).reshape(shp)
    x, B, C = arr("x", (b, L, H, P)), arr("B", (b, L, G, N)), arr("C", (b, L, G, N))
    dt, A, D = arr("dt", (b, L, H)), arr("A", (H,)), arr("D", (H,))
    init = None if case["init_state"] is None else arr("init_state", (b, H, P, N))
    out = _run(x, dt, A, B, C, D, init, T)
    tol = case["rel_tol"]
    np.testing.assert_allclose(out["y"].ravel(), case["expect_y"], rtol=tol,
                               atol=tol)
    np.testing.assert_allclose(out["states"].ravel(), case["expect_states"],
                               rtol=tol, atol=tol)
    np.testing.assert_allclose(out["final"].ravel(), case["expect_final"],
                               rtol=tol, atol=tol)
    g = oracle.chunk_cumsum(dt, A, T)
    np.testing.assert_allclose(g.ravel(), case["expect_g"], rtol=tol, atol=tol)


# --------------------------------------------------------- closed forms (C1,C2)
@pytest.mark.parametrize("T", [1, 4, 8, 16, 37])
def test_matches_chunked_closed_form(T):
    x, dt, A, B, C, D, init, _ = _rand_case(1)
    out = _run(x, dt, A, B, C, D, init, T)
    y, st, fin = chunked_form(x, dt, A, B, C, D, init, T)
    assert rel_err(out["y"], y) < 1e-12
    assert rel_err(out["states"], st) < 1e-12
    assert rel_err(out["final"], fin) < 1e-12


@pytest.mark.parametrize("seed,T,zero_init", [(2, 3, False), (3, 4, True),
                                              (4, 12, False)])
def test_matches_explicit_unrolling(seed, T, zero_init):
    x, dt, A, B, C, D, init, _ = _rand_case(seed, b=1, L=11, H=2, G=1, P=2,
                                            N=3, T=T, zero_init=zero_init)
    out = _run(x, dt, A, B, C, D, init, T)
    y, st, fin = unrolled_form(x, dt, A, B, C, D, init, T)
    assert rel_err(out["y"], y) < 1e-13
    assert rel_err(out["states"], st) < 1e-13
    assert rel_err(out["final"], fin) < 1e-13


# ------------------------------------------------------- special cases (C3,C4)
def test_no_decay_is_masked_matmul():
    x, dt, A, B, C, D, init, T = _rand_case(5, L=29, T=8)
    A = np.zeros_like(A)
    out = _run(x, dt, A, B, C, D, init, T)
    ref = masked_matmul_form(x, dt, B, C, D, init)
    assert rel_err(out["y"], ref) < 1e-13
    # the jump without decay: final = init + X^T (dt*B) summed over tokens
    b, L, H, P = x.shape
    hpg = H // B.shape[2]
    for bb in range(b):
        for h in range(H):
            Bw = dt[bb, :, h, None].astype(np.float64) * B[bb, :, h // hpg]
            fin = init[bb, h] + x[bb, :, h].astype(np.float64).T @ Bw
            assert rel_err(out["final"][bb, h], fin) < 1e-13


def test_unit_dt_no_decay_is_linear_attention():
    x, dt, A, B, C, D, init, T = _rand_case(6, L=20, T=4, zero_init=True)
    A = np.zeros_like(A)
    dt = np.ones_like(dt)
    out = _run(x, dt, A, B, C, D, None, T)
    b, L, H, P = x.shape
    hpg = H // B.shape[2]
    M = np.tril(np.ones((L, L)))
    for bb in range(b):
        for h in range(H):
            Cm = C[bb, :, h // hpg].astype(np.float64)
            Bm = B[bb, :, h // hpg].astype(np.float64)
            X = x[bb, :, h].astype(np.float64)
            ref = ((Cm @ Bm.T) * M) @ X + D[h] * X
            assert rel_err(out["y"][bb, :, h], ref) < 1e-13


def test_zero_dt_passes_state_through():
    x, dt, A, B, C, D, init, T = _rand_case(7, L=19, T=4)
    dt = np.zeros_like(dt)
    out = _run(x, dt, A, B, C, D, init, T)
    nc = out["states"].shape[2]
    for c in range(nc):
        assert np.array_equal(out["states"][:, :, c], init.astype(np.float64))
    assert np.array_equal(out["final"], init.astype(np.float64))
    b, L, H, P = x.shape
    hpg = H // B.shape[2]
    for bb in range(b):
        for h in range(H):
            ref = (C[bb, :, h // hpg].astype(np.float64)
                   @ init[bb, h].astype(np.float64).T
                   + D[h] * x[bb, :, h].astype(np.float64))
            assert rel_err(out["y"][bb, :, h], ref) < 1e-14
    g = oracle.chunk_cumsum(dt, A, T)
    assert np.all(g == 0)


# ------------------------------------------------------------ invariants (C5-C8)
@pytest.mark.parametrize("split", [16, 12])
def test_split_sequence_carries_state(split):
    x, dt, A, B, C, D, init, T = _rand_case(8, L=40, T=4)
    whole = _run(x, dt, A, B, C, D, init, T)
    first = _run(x[:, :split], dt[:, :split], A, B[:, :split], C[:, :split],
                 D, init, T)
    second = _run(x[:, split:], dt[:, split:], A, B[:, split:], C[:, split:],
                  D, first["final"], T)
    assert rel_err(np.concatenate([first["y"], second["y"]], 1),
                   whole["y"]) < 1e-12
    assert rel_err(second["final"], whole["final"]) < 1e-12
    if split % T == 0:
        st = np.concatenate([first["states"], second["states"]], 2)
        assert rel_err(st, whole["states"]) < 1e-12


def test_chunk_size_only_moves_sampling_points():
    x, dt, A, B, C, D, init, _ = _rand_case(9, L=48)
    runs = {T: _run(x, dt, A, B, C, D, init, T) for T in (1, 4, 16, 48)}
    for T, r in runs.items():
        assert rel_err(r["y"], runs[1]["y"]) < 1e-12
        assert rel_err(r["final"], runs[1]["final"]) < 1e-12
        # states at chunk c of size T are the T=1 states at token c*T
        assert rel_err(r["states"], runs[1]["states"][:, :, ::T]) < 1e-12


def test_bilinear_in_x_and_initial_state():
    x, dt, A, B, C, D, init, T = _rand_case(10, L=25, T=8)
    both = _run(x, dt, A, B, C, D, init, T)
    only_x = _run(x, dt, A, B, C, D, None, T)
    only_h = _run(np.zeros_like(x), dt, A, B, C, D, init, T)
    assert rel_err(only_x["y"] + only_h["y"], both["y"]) < 1e-12
    assert rel_err(only_x["final"] + only_h["final"], both["final"]) < 1e-12
    s = np.float32(0.5)
    scaled = _run(x * s, dt, A, B, C, D, init * s, T)
    assert rel_err(scaled["y"], 0.5 * both["y"]) < 1e-13
    zero = _run(np.zeros_like(x), dt, A, B, C, D, None, T)
    assert np.all(zero["y"] == 0) and np.all(zero["final"] == 0)


def test_extreme_decay_stays_finite_and_kept_weights_bounded():
    x, dt, A, B, C, D, init, T = _rand_case(11, L=32, T=8, a_scale=1e4)
    out = _run(x, dt, A, B, C, D, init, T)
    assert np.all(np.isfinite(out["y"]))
    assert np.all(np.isfinite(out["states"]))
    assert np.all(np.isfinite(out["final"]))
    # With total decay underflowing, each y_t is its own token's term only.
    b, L, H, P = x.shape
    hpg = H // B.shape[2]
    t, bb, h = 5, 0, 1
    g = h // hpg
    xt = x[bb, t, h].astype(np.float64)
    own = (float(dt[bb, t, h])
           * float(C[bb, t, g].astype(np.float64) @ B[bb, t, g].astype(np.float64))
           * xt + float(D[h]) * xt)
    assert rel_err(out["y"][bb, t, h], own) < 1e-12
    # kept pairwise weights 2^{g_i - g_j} (i >= j) are <= 1 because a <= 0
    gl = oracle.chunk_cumsum(dt, A, T)
    for c in range(L // T):
        seg = gl[:, :, c * T:(c + 1) * T]
        diff = seg[..., :, None] - seg[..., None, :]
        kept = np.tril(np.ones((T, T), bool))
        assert np.all(diff[..., kept] <= 0)


# ------------------------------------------------------------------ stage 1
def test_cumsum_exact_powers_of_two():
    # A = -1 and dt powers of two: every partial sum is exact in fp64, so
    # g = log2(e) * (-running sum) restarting at each chunk boundary.
    dt = np.array([0.5, 0.25, 1.0, 2.0, 0.125, 4.0, 0.5], np.float32)
    dt = np.tile(dt, (2, 3, 1)).transpose(0, 2, 1).copy()   # [2, 7, 3]
    A = np.array([-1.0, -2.0, -0.5], np.float32)
    T = 3
    g = oracle.chunk_cumsum(dt, A, T)
    log2e = 1.4426950408889634
    for h, a in enumerate(A):
        run, expect = 0.0, []
        for t in range(7):
            if t % T == 0:
                run = 0.0
            run += float(a) * float(dt[0, t, h])
            expect.append(run * log2e)
        np.testing.assert_array_equal(g[0, h], np.array(expect))
        np.testing.assert_array_equal(g[1, h], np.array(expect))


def test_cumsum_matches_decay_of_recurrence():
    # exp2 of the stage-1 output over a chunk equals the product of the
    # recurrence's own decay factors exp(A dt) over that chunk.
    x, dt, A, B, C, D, init, T = _rand_case(12, L=24, T=8)
    g = oracle.chunk_cumsum(dt, A, T)
    for c in range(3):
        prod = np.prod(np.exp(A[None, :].astype(np.float64)
                              * dt[:, c * T:(c + 1) * T].astype(np.float64)), 1)
        np.testing.assert_allclose(np.exp2(g[:, :, (c + 1) * T - 1]), prod,
                                   rtol=1e-13)


def test_pairs_subset_matches_full():
    x, dt, A, B, C, D, init, T = _rand_case(13, L=17, T=4)
    full = _run(x, dt, A, B, C, D, init, T)
    pairs = [5, 0, 3]
    sub = _run(x, dt, A, B, C, D, init, T, pairs=pairs)
    H = x.shape[2]
    for k, bh in enumerate(pairs):
        b, h = divmod(bh, H)
        assert np.array_equal(sub["y"][k], full["y"][b, :, h])
        assert np.array_equal(sub["states"][k], full["states"][b, h])
        assert np.array_equal(sub["final"][k], full["final"][b, h])


def test_chunk_out_from_own_states_reproduces_forward():
    x, dt, A, B, C, D, init, T = _rand_case(14, L=30, T=8)
    full = _run(x, dt, A, B, C, D, init, T)
    y = oracle.chunk_out(x, dt, A, B, C, D, full["states"], chunk_size=T)
    assert rel_err(y, full["y"]) < 1e-13
    # from arbitrary states with dt = 0 the output is C S_c^T + D x
    dt0 = np.zeros_like(dt)
    rng = np.random.default_rng(0)
    S = rng.standard_normal(full["states"].shape)
    y0 = oracle.chunk_out(x, dt0, A, B, C, D, S, chunk_size=T)
    b, L, H, P = x.shape
    hpg = H // B.shape[2]
    for t in (0, 7, 8, 29):
        c = t // T
        ref = (S[1, 2, c] @ C[1, t, 2 // hpg].astype(np.float64)
               + float(D[2]) * x[1, t, 2].astype(np.float64))
        np.testing.assert_allclose(y0[1, t, 2], ref, rtol=1e-13, atol=1e-13)


def test_named_workload_small_variant_runs():
    # the full tiny workload is small enough for all three pins at once
    w = WORKLOADS["tiny_fp32"]
    inp = make_inputs(w)
    out = _run(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
               inp["init_state"], w.chunk_size)
    y, st, fin = chunked_form(inp["x"], inp["dt"], inp["A"], inp["B"],
                              inp["C"], inp["D"], inp["init_state"],
                              w.chunk_size)
    assert rel_err(out["y"], y) < 1e-12
    assert rel_err(out["states"], st) < 1e-12
    assert rel_err(out["final"], fin) < 1e-12
