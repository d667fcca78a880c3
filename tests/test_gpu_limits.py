"""The hot path at the largest sizes the C ABI accepts.

* ssd_forward on one (batch, head) whose sequence is the longest a chunk of
  256 allows for P = N = 64: (L + T) * H * P * 4 bytes must stay below 2^31,
  so L = 2^23 - 256 - 1 tokens (32767 chunks, the last one 255 tokens).  One
  token more is rejected.  The same on one head pair with N = 128 and
  128-token chunks (L = 2^22 - 128 - 1), which takes the bf16 fused pass.  Inputs are drawn on the device from a seeded
  generator with the distributions of the workloads.  Checked against the
  fp64 oracle on the first 16 chunks (states and y depend on the prefix
  only), and at the end through the split property the oracle is pinned
  to: the last two chunks run again from the big run's state at their start
  must give its y, states and final state (to the bf16 arithmetic bound;
  the two runs take different state-pass kernels).
* ssd_causal_conv1d on the longest row it accepts (2^29 - 2^14 tokens, one
  channel, bf16 in and out), compared with the oracle on windows at the
  start, the middle and the end of the row (out[t] depends on x[t-3 .. t]).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _gen(seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return g


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _longest_forward(ssd, T, N, H, G, seed):
    """ssd_forward on one batch row at the longest sequence the per-sequence
    extent rule allows for (T, N, H, G); checked as the module docstring
    describes."""
    P = 64
    L = (1 << 31) // (H * P * 4) - T - 1
    # the library sizes the workspace for L and refuses L + 1 (0 = invalid)
    ws = ssd.workspace_bytes(ssd.SsdDims(1, L, H, P, N, G, T))
    assert ws == 8 * L * H
    assert ssd.workspace_bytes(ssd.SsdDims(1, L + 1, H, P, N, G, T)) == 0
    log(f"[limits] ssd_forward b=1 L={L} H={H} P={P} N={N} G={G} T={T}")
    gen = _gen(seed)
    bf = torch.bfloat16
    x = torch.randn(1, L, H, P, device=DEV, generator=gen).to(bf)
    B = torch.randn(1, L, G, N, device=DEV, generator=gen).to(bf)
    C = torch.randn(1, L, G, N, device=DEV, generator=gen).to(bf)
    dt = torch.nn.functional.softplus(
        torch.randn(1, L, H, device=DEV, generator=gen, dtype=torch.float64) - 2.0).float()
    A = -torch.exp(torch.rand(H, device=DEV, generator=gen, dtype=torch.float64) * 1.5).float()
    D = torch.randn(H, device=DEV, generator=gen)
    init = 0.1 * torch.randn(1, H, P, N, device=DEV, generator=gen)
    y, states, final = ssd.forward(x, dt, A, B, C, D, init, chunk_size=T)
    torch.cuda.synchronize()
    nc = states.shape[2]
    assert nc == 32767 and L % T == T - 1
    for name, t in (("y", y), ("states", states), ("final", final)):
        assert bool(torch.isfinite(t).all()), name

    # the first 16 chunks against the oracle
    Lp = 16 * T
    ref = oracle.forward(_np(x[:, :Lp]), _np(dt[:, :Lp]), _np(A), _np(B[:, :Lp]),
                         _np(C[:, :Lp]), _np(D), _np(init), chunk_size=T)
    assert_close(_np(y[:, :Lp]), ref["y"], "bf16", "y (prefix)")
    assert_close(_np(states[:, :, :16]), ref["states"], "bf16", "states (prefix)")

    # the last two chunks again, from the big run's state at their start
    ts = (nc - 2) * T
    y2, st2, fin2 = ssd.forward(x[:, ts:].contiguous(), dt[:, ts:].contiguous(), A,
                                B[:, ts:].contiguous(), C[:, ts:].contiguous(), D,
                                states[:, :, nc - 2].contiguous(), chunk_size=T)
    torch.cuda.synchronize()
    assert torch.equal(st2[:, :, 0], states[:, :, nc - 2])
    for what, got, want in (("states (tail)", st2[:, :, 1], states[:, :, nc - 1]),
                            ("final (tail)", fin2, final), ("y (tail)", y2, y[:, ts:])):
        g_, w_ = _np(got), _np(want)
        e = float(np.max(np.abs(g_ - w_)) / np.sqrt(np.mean(w_ ** 2)))
        log(f"  {what}: max|d|/RMS={e:.3e}")
        assert e <= 2e-3, (what, e)


def test_forward_at_the_longest_sequence(ssd):
    # one head, N = 64: the stage kernels (the two-level state pass)
    _longest_forward(ssd, T=256, N=64, H=1, G=1, seed=31)


def test_forward_at_the_longest_sequence_bf16_fused_pass(ssd):
    # one head pair, N = 128: the bf16 fused pass, its chain cut into 256
    # runs of 128 chunks (4 194 175 tokens, 2 GiB of states)
    _longest_forward(ssd, T=128, N=128, H=2, G=1, seed=33)


def test_conv1d_at_the_longest_row(ssd):
    L = (1 << 29) - (1 << 14)
    W = 4
    log(f"[limits] ssd_causal_conv1d b=1 dim=1 L={L} W={W} bf16")
    gen = _gen(32)
    x = torch.randn(1, 1, L, device=DEV, generator=gen).to(torch.bfloat16)
    w = torch.randn(1, W, device=DEV, generator=gen) * 0.5
    bias = torch.randn(1, device=DEV, generator=gen)
    out = torch.empty_like(x)
    ssd.ssd_causal_conv1d(x, w, bias, out)
    torch.cuda.synchronize()
    wn, bn = _np(w), _np(bias)
    for s in (0, L // 2 - 777, L - 4096):
        e = s + 4096
        lo = max(s - (W - 1), 0)
        xs = _np(x[:, :, lo:e])
        ref = oracle.causal_conv1d(xs, wn, bn)[:, :, s - lo:]
        S = oracle.causal_conv1d(np.abs(xs), np.abs(wn), np.abs(bn))[:, :, s - lo:]
        bound = (W + 2) * 2.0 ** -24 * S
        bound = bound + 2.0 ** -8 * (np.abs(ref) + bound)
        got = _np(out[:, :, s:e])
        assert np.all(np.isfinite(got))
        err = np.abs(got - ref)
        log(f"  window at {s}: max|d|/bound={float(np.max(err / bound)):.3f}")
        assert np.all(err <= bound), s
