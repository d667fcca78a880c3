"""Independent fp64 numpy forms used to pin the oracle (test helpers).

None of these re-types the oracle's token loop.  Each is a different
statement of the same mathematics, taken from the pages:

* ``chunked_form`` -- the chunkwise identities ("Accelerating Mamba-2 with
  High-Performance Forward Pass Kernels in NVIDIA CUDA Tile", sections
  "Step 1: Jump the State Across a Chunk with One Matmul" and "Step 3: Add
  Back the Decay, Safely, in Log-Space"; written out on the zhiding.cn
  rendering, section "Mamba-2架构"): with G the within-chunk cumsum of a,
    h_next = e^{G_last} h + (e^{G_last - G} * dt * B)^T X   (as [P, N]: X^T ...)
    Y      = e^{G} (C h^T) + ((C B^T) * e^{G_i - G_j} * M) (dt * X) + D X
  using natural exp, matrix products and a mask.
* ``unrolled_form`` -- the closed-form unrolling of the recurrence with
  explicit products of decay factors (no cumsums), for tiny inputs.
* ``masked_matmul_form`` -- the decay-free case, which the pages identify as
  linear attention: Y = ((C (dt*B)^T) * M) X + D X + C h0^T
  (section "Step 2: Compute a Chunk of Outputs from One State").
"""
from __future__ import annotations

import numpy as np


def chunked_form(x, dt, A, B, C, D, init, T):
    """Returns y [b,L,H,P], states [b,H,nc,P,N], final [b,H,P,N] (fp64)."""
    x, dt, A, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    nc = -(-L // T)
    y = np.zeros((b, L, H, P))
    states = np.zeros((b, H, nc, P, N))
    final = np.zeros((b, H, P, N))
    for bb in range(b):
        for h in range(H):
            g = h // hpg
            S = (np.zeros((P, N)) if init is None
                 else np.asarray(init[bb, h], np.float64).copy())
            for c in range(nc):
                states[bb, h, c] = S
                sl = slice(c * T, min((c + 1) * T, L))
                X = x[bb, sl, h]            # [t, P]
                Bm = B[bb, sl, g]           # [t, N]
                Cm = C[bb, sl, g]           # [t, N]
                d = dt[bb, sl, h]           # [t]
                Gc = np.cumsum(A[h] * d)    # inclusive, natural-log units
                n = len(d)
                ii, jj = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
                expo = np.where(ii >= jj, Gc[:, None] - Gc[None, :], -np.inf)
                Lmat = (Cm @ Bm.T) * np.exp(expo)
                Y = (np.exp(Gc)[:, None] * (Cm @ S.T)
                     + Lmat @ (d[:, None] * X) + D[h] * X)
                y[bb, sl, h] = Y
                w = np.exp(Gc[-1] - Gc) * d
                S = np.exp(Gc[-1]) * S + X.T @ (w[:, None] * Bm)
            final[bb, h] = S
    return y, states, final


def unrolled_form(x, dt, A, B, C, D, init, T):
    """Explicit-product unrolling; O(L^2 P N) per head: tiny inputs only.

    y_t = sum_{s<=t} (prod_{k=s+1..t} e^{a_k}) dt_s (C_t . B_s) x_s
          + (prod_{k=0..t} e^{a_k}) h0 C_t + D x_t
    states[c] = sum_{s<cT} (prod_{k=s+1..cT-1} e^{a_k}) dt_s x_s B_s^T
                + (prod_{k=0..cT-1} e^{a_k}) h0
    """
    x, dt, A, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    nc = -(-L // T)
    y = np.zeros((b, L, H, P))
    states = np.zeros((b, H, nc, P, N))
    final = np.zeros((b, H, P, N))

    for bb in range(b):
        for h in range(H):
            g = h // hpg
            h0 = (np.zeros((P, N)) if init is None
                  else np.asarray(init[bb, h], np.float64))
            e = np.exp(A[h] * dt[bb, :, h])   # per-token decay factors

            def prod(lo, hi):   # product of e[k] for k in [lo, hi]
                r = 1.0
                for k in range(lo, hi + 1):
                    r *= e[k]
                return r

            def state_before(t):   # state after tokens 0..t-1
                S = prod(0, t - 1) * h0
                for s in range(t):
                    S = S + prod(s + 1, t - 1) * dt[bb, s, h] * np.outer(
                        x[bb, s, h], B[bb, s, g])
                return S

            for t in range(L):
                acc = prod(0, t) * (h0 @ C[bb, t, g])
                for s in range(t + 1):
                    acc = acc + (prod(s + 1, t) * dt[bb, s, h]
                                 * float(C[bb, t, g] @ B[bb, s, g])) * x[bb, s, h]
                y[bb, t, h] = acc + D[h] * x[bb, t, h]
            for c in range(nc):
                states[bb, h, c] = state_before(c * T)
            final[bb, h] = state_before(L)
    return y, states, final


def masked_matmul_form(x, dt, B, C, D, init):
    """Decay-free (A = 0) output over the whole sequence as a masked matmul."""
    x, dt, B, C, D = (np.asarray(v, np.float64) for v in (x, dt, B, C, D))
    b, L, H, P = x.shape
    G = B.shape[2]
    hpg = H // G
    M = np.tril(np.ones((L, L)))
    y = np.zeros((b, L, H, P))
    for bb in range(b):
        for h in range(H):
            g = h // hpg
            Bw = dt[bb, :, h][:, None] * B[bb, :, g]
            Y = ((C[bb, :, g] @ Bw.T) * M) @ x[bb, :, h] + D[h] * x[bb, :, h]
            if init is not None:
                Y = Y + C[bb, :, g] @ np.asarray(init[bb, h], np.float64).T
            y[bb, :, h] = Y
    return y


def rel_err(got, ref):
    """max |got - ref| / max(|ref|, RMS(ref)) elementwise (RMS-floored)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den)) if ref.size else 0.0


def rms_err(got, ref):
    """max |got - ref| / RMS(ref)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    if rms == 0:
        return float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return float(np.max(np.abs(got - ref)) / rms)
