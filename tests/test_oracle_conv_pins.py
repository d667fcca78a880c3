"""Pins of the oracle's causal depthwise conv1d (CPU only).

out[b,d,t] = bias[d] + sum_k weight[d,k] x[b,d,t-W+1+k], zero left padding
(page 3, the Helion hackathon gallery, its causal_conv1d entries).  The pins:
the impulse response (which tap lands where), numpy's convolution (an
independent implementation of the same sum), the constant-input closed form
(the causal edge), causality and linearity.
"""
import numpy as np
import pytest

import oracle


def _case(seed, b=2, d=5, L=23, W=4, bias=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((b, d, L)).astype(np.float32)
    w = rng.standard_normal((d, W)).astype(np.float32)
    bb = rng.standard_normal(d).astype(np.float32) if bias else None
    return x, w, bb


@pytest.mark.parametrize("W", [2, 3, 4])
def test_impulse_response_places_taps_in_reverse(W):
    L, t0 = 12, 5
    x = np.zeros((1, 3, L), np.float32)
    x[0, 1, t0] = 1.0
    w = np.arange(1, 3 * W + 1, dtype=np.float32).reshape(3, W)
    bias = np.array([0.0, -0.5, 0.0], np.float32)
    out = oracle.causal_conv1d(x, w, bias)
    expect = np.full(L, -0.5)
    for j in range(W):                       # out[t0 + j] takes tap W-1-j
        expect[t0 + j] += w[1, W - 1 - j]
    np.testing.assert_array_equal(out[0, 1], expect)
    assert np.all(out[0, 0] == 0) and np.all(out[0, 2] == 0)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_matches_numpy_convolution(W):
    x, w, bias = _case(1, W=W)
    out = oracle.causal_conv1d(x, w, bias)
    ref = np.empty_like(out)
    for b in range(x.shape[0]):
        for d in range(x.shape[1]):
            full = np.convolve(x[b, d].astype(np.float64), w[d, ::-1].astype(np.float64))
            ref[b, d] = full[: x.shape[2]] + bias[d]
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_constant_input_causal_edge():
    W, L, c = 4, 9, 2.5
    x = np.full((1, 2, L), c, np.float32)
    w = np.array([[1, 2, 3, 4], [0.5, -1, 0, 2]], np.float32)
    out = oracle.causal_conv1d(x, w, None)
    for d in range(2):
        for t in range(L):
            # taps k >= W-1-t see the signal; earlier ones see the padding
            expect = c * sum(float(w[d, k]) for k in range(max(0, W - 1 - t), W))
            assert out[0, d, t] == pytest.approx(expect, abs=1e-12)


def test_causal_and_local():
    x, w, bias = _case(2, L=20)
    base = oracle.causal_conv1d(x, w, bias)
    x2 = x.copy()
    s = 11
    x2[1, 3, s] += 7.0
    out = oracle.causal_conv1d(x2, w, bias)
    diff = out - base
    changed = np.nonzero(np.abs(diff) > 0)
    assert set(changed[0]) == {1} and set(changed[1]) == {3}
    ts = changed[2]
    assert ts.min() >= s and ts.max() < s + w.shape[1]


def test_linear_in_x_without_bias():
    x, w, _ = _case(3, bias=False)
    y, _, _ = _case(4, bias=False)
    a, b = 0.75, -1.5
    lhs = oracle.causal_conv1d((a * x + b * y).astype(np.float64).astype(np.float32), w)
    # float32 rounding of the combined input is the only difference
    rhs = a * oracle.causal_conv1d(x, w) + b * oracle.causal_conv1d(y, w)
    assert np.max(np.abs(lhs - rhs)) < 1e-5 * max(1.0, np.max(np.abs(rhs)))


def test_shorter_than_filter():
    x, w, bias = _case(5, L=2, W=4)
    out = oracle.causal_conv1d(x, w, bias)
    for t in range(2):
        expect = bias[None, :] + sum(w[None, :, 4 - 1 - j] * x[:, :, t - j]
                                     for j in range(t + 1))
        np.testing.assert_allclose(out[:, :, t], expect, rtol=1e-6, atol=1e-6)
