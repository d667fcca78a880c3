"""Pins of the oracle's Gated DeltaNet chunked forward (CPU only).

The oracle runs the gallery's per-chunk steps (page 3, the Helion hackathon
gallery, gated_deltanet_chunk_fwd_h / chunk_fwd_o): store h, v_new = u - w h,
gate v_new by exp(g_last - g_t), decay h by exp(g_last), add k^T v_gated;
o = exp(g) q h + causal(q k^T exp(g_i - g_j)) v_new.  Those steps are pinned
here against things other than themselves:

* The token-by-token gated delta rule, S_t = a_t (I - b_t k_t k_t^T) S_{t-1}
  + b_t k_t v_t^T, o_t = S_t^T q_t, written out in numpy.  When w and u come
  from the WY transform of (k, v, beta, g) -- w = T (beta exp(g) k), u =
  T (beta v), T = (I + strictly-lower(diag(beta) K K^T o exp(g_i - g_j)))^-1,
  the gallery's recompute_w_u entries -- the chunked steps must reproduce the
  token recurrence exactly (up to rounding).  Any dropped term, wrong sign,
  wrong gate index or transposed operand in either oracle function breaks it.
* With w = 0 the delta correction vanishes and the pass is gated linear
  attention: a brute-force double sum with explicit products of the gates,
  and the result must not depend on the chunk size (the chunk bookkeeping,
  including the ragged last chunk, is pinned by that).
* Exact special cases: the first stored state is h0; zero inputs give zeros.
"""
import numpy as np
import pytest

import oracle


def _chunk_cumsum(a, C):
    """Chunk-local inclusive cumsum along axis 1 of a [b, L, H] (float64)."""
    g = np.zeros_like(a, dtype=np.float64)
    L = a.shape[1]
    for t0 in range(0, L, C):
        g[:, t0:t0 + C] = np.cumsum(a[:, t0:t0 + C].astype(np.float64), axis=1)
    return g


def _inputs(seed, b, L, H, K, V, C):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((b, L, H, K)).astype(np.float32)
    k = rng.standard_normal((b, L, H, K))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((b, L, H, V)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, size=(b, L, H)).astype(np.float32)
    a = rng.uniform(-0.6, -0.01, size=(b, L, H))
    g = _chunk_cumsum(a, C).astype(np.float32)
    h0 = rng.standard_normal((b, H, K, V)) * 0.5
    return q, k, v, beta, g, h0


def _token_gates(g, C):
    """Per-token log-gates recovered from the (float32) chunk-local g."""
    g = g.astype(np.float64)
    a = g.copy()
    L = g.shape[1]
    for t in range(L):
        if t % C:
            a[:, t] = g[:, t] - g[:, t - 1]
    return a


def _wy(k, v, beta, g, C):
    """w, u of every chunk from the WY transform, in float64."""
    b, L, H, K = k.shape
    V = v.shape[3]
    w = np.zeros((b, L, H, K))
    u = np.zeros((b, L, H, V))
    for bb in range(b):
        for h in range(H):
            for t0 in range(0, L, C):
                t1 = min(t0 + C, L)
                kc = k[bb, t0:t1, h].astype(np.float64)
                vc = v[bb, t0:t1, h].astype(np.float64)
                bc = beta[bb, t0:t1, h].astype(np.float64)
                gc = g[bb, t0:t1, h].astype(np.float64)
                n = t1 - t0
                M = np.eye(n)
                for i in range(n):
                    for j in range(i):
                        M[i, j] = bc[i] * (kc[i] @ kc[j]) * np.exp(gc[i] - gc[j])
                Tm = np.linalg.inv(M)
                u[bb, t0:t1, h] = Tm @ (bc[:, None] * vc)
                w[bb, t0:t1, h] = Tm @ ((bc * np.exp(gc))[:, None] * kc)
    return w, u


def _token_recurrence(q, k, v, beta, a, h0, scale):
    b, L, H, K = q.shape
    V = v.shape[3]
    o = np.zeros((b, L, H, V))
    fin = np.zeros((b, H, K, V))
    for bb in range(b):
        for h in range(H):
            S = h0[bb, h].astype(np.float64).copy()
            for t in range(L):
                kt = k[bb, t, h].astype(np.float64)
                alpha = np.exp(a[bb, t, h])
                bt = float(beta[bb, t, h])
                S = alpha * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[bb, t, h])
                o[bb, t, h] = scale * (S.T @ q[bb, t, h].astype(np.float64))
            fin[bb, h] = S
    return o, fin


@pytest.mark.parametrize("L,C", [(11, 4), (16, 8), (7, 64)])
def test_chunked_steps_reproduce_the_gated_delta_rule(L, C):
    b, H, K, V, scale = 2, 2, 5, 3, 0.7
    q, k, v, beta, g, h0 = _inputs(10 + L, b, L, H, K, V, C)
    w, u = _wy(k, v, beta, g, C)
    st = oracle.gdn_chunk_fwd_h(k, w.astype(np.float32), u.astype(np.float32), g, h0,
                                chunk_size=C)
    o = oracle.gdn_chunk_fwd_o(q, k, st["v_new"], st["h"], g, scale=scale, chunk_size=C)
    o_ref, fin_ref = _token_recurrence(q, k, v, beta, _token_gates(g, C), h0, scale)
    # w and u enter the oracle rounded to float32: relative error ~1e-7
    np.testing.assert_allclose(st["final"], fin_ref, rtol=2e-5, atol=2e-5)
    np.testing.assert_allclose(o, o_ref, rtol=2e-5, atol=2e-5)


def test_without_delta_term_is_gated_linear_attention():
    """w = 0: v_new = u and the state is a gated sum of k u^T; the output is
    gated linear attention.  Brute force with explicit products of gates."""
    b, L, H, K, V, C = 1, 13, 2, 4, 3, 5
    q, k, v, beta, g, h0 = _inputs(3, b, L, H, K, V, C)
    a = _token_gates(g, C)
    u = v
    u64, k64 = u.astype(np.float64), k.astype(np.float64)
    w = np.zeros_like(k)
    st = oracle.gdn_chunk_fwd_h(k, w, u, g, h0, chunk_size=C)
    o = oracle.gdn_chunk_fwd_o(q, k, st["v_new"], st["h"], g, chunk_size=C)
    for h in range(H):
        for t in range(L):
            ref = np.prod(np.exp(a[0, : t + 1, h])) * (q[0, t, h].astype(np.float64)
                                                      @ h0[0, h])
            for s in range(t + 1):
                gate = np.prod(np.exp(a[0, s + 1: t + 1, h]))
                ref = ref + gate * float(q[0, t, h].astype(np.float64)
                                         @ k64[0, s, h]) * u64[0, s, h]
            np.testing.assert_allclose(o[0, t, h], ref, rtol=1e-12, atol=1e-12)
        fin = np.prod(np.exp(a[0, :, h])) * h0[0, h]
        for s in range(L):
            gate = np.prod(np.exp(a[0, s + 1:, h]))
            fin = fin + gate * np.outer(k64[0, s, h], u64[0, s, h])
        np.testing.assert_allclose(st["final"][0, h], fin, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(st["v_new"], u.astype(np.float64))


def test_without_delta_term_chunk_size_does_not_matter():
    b, L, H, K, V = 2, 23, 2, 4, 6
    q, k, v, beta, _, h0 = _inputs(4, b, L, H, K, V, 1)
    rng = np.random.default_rng(5)
    a = rng.uniform(-0.4, -0.01, size=(b, L, H)).astype(np.float32)
    w = np.zeros_like(k)
    outs = []
    for C in (1, 4, 7, 64):
        g = _chunk_cumsum(a, C)   # float64: g must match the same gates exactly
        st = oracle.gdn_chunk_fwd_h(k, w, v, g, h0, chunk_size=C)
        outs.append((oracle.gdn_chunk_fwd_o(q, k, st["v_new"], st["h"], g, chunk_size=C),
                     st["final"]))
    for o, f in outs[1:]:
        # g is rounded to float32 differently per chunking: ~1e-6 relative
        np.testing.assert_allclose(o, outs[0][0], rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(f, outs[0][1], rtol=1e-5, atol=1e-5)


def test_first_state_is_h0_and_zeros_stay_zero():
    b, L, H, K, V, C = 1, 9, 1, 3, 2, 4
    q, k, v, beta, g, h0 = _inputs(6, b, L, H, K, V, C)
    w, u = _wy(k, v, beta, g, C)
    st = oracle.gdn_chunk_fwd_h(k, w, u, g, h0, chunk_size=C)
    np.testing.assert_array_equal(st["h"][:, :, 0], h0)
    z = oracle.gdn_chunk_fwd_h(k, w, np.zeros_like(u), g, None, chunk_size=C)
    assert not np.any(z["h"]) and not np.any(z["v_new"]) and not np.any(z["final"])
    o = oracle.gdn_chunk_fwd_o(q, k, z["v_new"], z["h"], g, chunk_size=C)
    assert not np.any(o)
