"""Parity of the Gated DeltaNet chunked forward (ssd_gdn_chunk_fwd_h and
ssd_gdn_chunk_fwd_o, through the C ABI) with the fp64 oracle.

Tolerances are the bf16-input ones of the SSD path: max |d| / RMS(ref) <=
2e-2, and the tighter 2e-3 the arithmetic supports (exact bf16 inputs, the
fp32 state and every other computed operand split into bf16 hi + lo, fp32
accumulation).  Outputs rounded to bf16 (v_new, o) are held to the
RMS-floored relative bound 1e-2.

Cases span both workgroup widths (two and four waves), K and V of 64 and 128,
ragged last chunks, a carried-in initial state, and the benchmark layer at
full size on sampled (batch, head) pairs.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_close, log
from ssd_workloads import GDN_WORKLOADS, GdnWorkload, make_gdn_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


def _dev(inp, key, dtype=torch.bfloat16):
    a = inp[key]
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV, dtype)


def _np(t):
    return t.detach().float().cpu().numpy()


def _run_h(ssd, c, inp, vdt=torch.float32):
    k, w, u = _dev(inp, "k"), _dev(inp, "w"), _dev(inp, "u")
    g = _dev(inp, "g", torch.float32)
    h0 = _dev(inp, "h0", torch.float32)
    b, L, H, K, V = c.batch, c.seqlen, c.nheads, c.dk, c.dv
    h = torch.full((b, H, c.nchunks, K, V), float("nan"), device=DEV)
    vn = torch.full((b, L, H, V), float("nan"), device=DEV, dtype=vdt)
    fin = torch.full((b, H, K, V), float("nan"), device=DEV)
    ssd.ssd_gdn_chunk_fwd_h(k, w, u, g, h0, h, vn, fin)
    torch.cuda.synchronize()
    return h, vn, fin


H_CASES = [
    # b, L, H, K, V, init
    (1, 200, 2, 64, 64, 0.3),      # ragged last chunk, two waves
    (2, 130, 3, 128, 64, None),
    (1, 64, 2, 64, 128, 0.2),      # one chunk
    (2, 129, 2, 128, 128, 0.1),    # ragged by one token
    (2, 70, 64, 128, 128, None),   # 256 workgroups of four waves
    (1, 1, 2, 128, 128, 0.5),      # a single token
]


@pytest.mark.parametrize("b,L,H,K,V,init", H_CASES,
                         ids=[f"b{c[0]}_L{c[1]}_H{c[2]}_K{c[3]}_V{c[4]}" + ("_init" if c[5] else "")
                              for c in H_CASES])
def test_fwd_h_matches_oracle(ssd, b, L, H, K, V, init):
    c = GdnWorkload("gdn_case", b, L, H, K, V, "bf16", init)
    inp = make_gdn_inputs(c, seed=50 + L)
    log(f"[gdn h] b={b} L={L} H={H} K={K} V={V} init={init}")
    h, vn, fin = _run_h(ssd, c, inp)
    ref = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    assert_close(_np(h), ref["h"], "bf16", "h")
    assert_close(_np(vn), ref["v_new"], "bf16", "v_new")
    assert_close(_np(fin), ref["final"], "bf16", "final")


def test_fwd_h_bf16_v_new(ssd):
    c = GdnWorkload("gdn_case", 2, 150, 2, 128, 128, "bf16", 0.2)
    inp = make_gdn_inputs(c, seed=61)
    h, vn, fin = _run_h(ssd, c, inp, torch.bfloat16)
    ref = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    assert_close(_np(vn), ref["v_new"], "bf16", "v_new (bf16)", y_bf16=True)
    assert_close(_np(h), ref["h"], "bf16", "h")


def test_fwd_h_layer_full_size_sampled(ssd):
    """The benchmark layer at full size, as the benchmark launches it; the
    oracle runs on sampled (batch, head) pairs."""
    c = GDN_WORKLOADS["gdn_layer_bf16"]
    inp = make_gdn_inputs(c, seed=3)
    log(f"[gdn h] full size {c}")
    h, vn, fin = _run_h(ssd, c, inp, torch.bfloat16)
    assert torch.isfinite(h).all() and torch.isfinite(fin).all()
    for (bi, hi) in [(0, 0), (3, 7), (7, 15), (5, 2)]:
        sub = {k: (None if v is None else v[bi:bi + 1, :, hi:hi + 1]) for k, v in inp.items()
               if k in ("k", "w", "u", "g")}
        ref = oracle.gdn_chunk_fwd_h(sub["k"], sub["w"], sub["u"], sub["g"], None)
        assert_close(_np(h[bi, hi]), ref["h"][0, 0], "bf16", f"h[{bi},{hi}]")
        assert_close(_np(fin[bi, hi]), ref["final"][0, 0], "bf16", f"final[{bi},{hi}]")
        assert_close(_np(vn[bi, :, hi]), ref["v_new"][0, :, 0], "bf16", f"v_new[{bi},{hi}]",
                     y_bf16=True)


def test_fwd_h_zero_values_give_zero(ssd):
    c = GdnWorkload("gdn_case", 1, 100, 2, 64, 64, "bf16", None)
    inp = make_gdn_inputs(c, seed=62)
    inp["u"] = np.zeros_like(inp["u"])
    h, vn, fin = _run_h(ssd, c, inp)
    assert not torch.any(h) and not torch.any(vn) and not torch.any(fin)


def test_fwd_h_rejects_bad_arguments(ssd):
    c = GdnWorkload("gdn_case", 1, 64, 2, 64, 64, "bf16", None)
    inp = make_gdn_inputs(c, seed=63)
    k, w, u = _dev(inp, "k"), _dev(inp, "w"), _dev(inp, "u")
    g = _dev(inp, "g", torch.float32)
    h = torch.empty(1, 2, 1, 64, 64, device=DEV)
    vn = torch.empty(1, 64, 2, 64, device=DEV)
    with pytest.raises(ValueError):
        ssd.ssd_gdn_chunk_fwd_h(k, w, u, g, None, h[:, :1].contiguous(), vn, None)
    with pytest.raises(TypeError):
        ssd.ssd_gdn_chunk_fwd_h(k, w.float(), u, g, None, h, vn, None)
    with pytest.raises(ssd.SsdError):   # fp32 inputs are not built
        ssd.ssd_gdn_chunk_fwd_h(k.float(), w.float(), u.float(), g, None, h, vn, None)


def _run_o(ssd, c, inp, vn, h, odt=torch.float32, scale=1.0):
    q, k = _dev(inp, "q"), _dev(inp, "k")
    g = _dev(inp, "g", torch.float32)
    o = torch.full((c.batch, c.seqlen, c.nheads, c.dv), float("nan"), device=DEV, dtype=odt)
    ssd.ssd_gdn_chunk_fwd_o(q, k, vn, h, g, o, scale)
    torch.cuda.synchronize()
    return o


O_CASES = [
    # b, L, H, K, V, scale
    (1, 200, 2, 64, 64, 1.0),
    (2, 130, 3, 128, 64, 0.5),
    (1, 64, 2, 64, 128, 1.0),
    (2, 129, 2, 128, 128, 0.0883883),
    (1, 1, 2, 128, 128, 1.0),
    # more items than resident workgroups: runs of one or two items that start
    # at either column block of a head (k and q loaded or reused)
    (5, 640, 10, 128, 128, 1.0),
    (4, 1100, 12, 64, 64, 0.5),
]


@pytest.mark.parametrize("b,L,H,K,V,scale", O_CASES,
                         ids=[f"b{c[0]}_L{c[1]}_H{c[2]}_K{c[3]}_V{c[4]}_s{c[5]}" for c in O_CASES])
def test_fwd_o_alone_matches_oracle(ssd, b, L, H, K, V, scale):
    """chunk_fwd_o fed the oracle's states and its v_new rounded to bf16; the
    oracle output is computed from exactly those values."""
    c = GdnWorkload("gdn_case", b, L, H, K, V, "bf16", 0.2)
    inp = make_gdn_inputs(c, seed=70 + L)
    log(f"[gdn o] b={b} L={L} H={H} K={K} V={V} scale={scale}")
    ref_h = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    vn = torch.from_numpy(ref_h["v_new"].astype(np.float32)).to(DEV, torch.bfloat16)
    h = torch.from_numpy(ref_h["h"].astype(np.float32)).to(DEV)
    o = _run_o(ssd, c, inp, vn, h, scale=scale)
    ref = oracle.gdn_chunk_fwd_o(inp["q"], inp["k"], _np(vn).astype(np.float64),
                                 _np(h).astype(np.float64), inp["g"], scale=scale)
    assert_close(_np(o), ref, "bf16", "o")


@pytest.mark.parametrize("K,V", [(64, 64), (128, 128)])
def test_fwd_h_then_o_match_oracle_chain(ssd, K, V):
    """The two kernels in sequence (v_new handed over in bf16) against the
    oracle's fp64 chain, element by element.  Rounding v_new to bf16 moves
    each v_new[j] by at most 2^-8 |v_new[j]|, so o[t] moves by at most
    2^-8 sum_j |q_t . k_j| e^{g_t - g_j} |v_new[j]| <= 2^-8 S[t], with S the
    oracle output on |q|, |k|, |v_new| and no state term.  The rest of the
    arithmetic (fp32 with split operands) adds 1e-3 RMS(o) of slack."""
    c = GdnWorkload("gdn_case", 2, 190, 3, K, V, "bf16", 0.3)
    inp = make_gdn_inputs(c, seed=80 + K)
    h, vn, fin = _run_h(ssd, c, inp, torch.bfloat16)
    o = _run_o(ssd, c, inp, vn, h)
    ref_h = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    ref = oracle.gdn_chunk_fwd_o(inp["q"], inp["k"], ref_h["v_new"], ref_h["h"], inp["g"])
    S = oracle.gdn_chunk_fwd_o(np.abs(inp["q"]), np.abs(inp["k"]), np.abs(ref_h["v_new"]),
                               np.zeros_like(ref_h["h"]), inp["g"])
    got = _np(o).astype(np.float64)
    bound = 2.0 ** -8 * S + 1e-3 * np.sqrt(np.mean(ref ** 2))
    worst = float(np.max(np.abs(got - ref) / bound))
    log(f"  o (chain, bf16 v_new between kernels): max|d|/bound={worst:.3f}")
    assert np.all(np.isfinite(got)) and worst <= 1.0


def test_fwd_o_bf16_output(ssd):
    c = GdnWorkload("gdn_case", 1, 150, 2, 128, 128, "bf16", 0.2)
    inp = make_gdn_inputs(c, seed=90)
    ref_h = oracle.gdn_chunk_fwd_h(inp["k"], inp["w"], inp["u"], inp["g"], inp["h0"])
    vn = torch.from_numpy(ref_h["v_new"].astype(np.float32)).to(DEV, torch.bfloat16)
    h = torch.from_numpy(ref_h["h"].astype(np.float32)).to(DEV)
    o = _run_o(ssd, c, inp, vn, h, odt=torch.bfloat16)
    ref = oracle.gdn_chunk_fwd_o(inp["q"], inp["k"], _np(vn).astype(np.float64),
                                 _np(h).astype(np.float64), inp["g"])
    assert_close(_np(o), ref, "bf16", "o (bf16)", y_bf16=True)


def test_fwd_o_layer_full_size_sampled(ssd):
    """The benchmark layer at full size (both kernels, as the benchmark runs
    them); sampled (batch, head) pairs against the oracle on the kernel's own
    h and v_new."""
    c = GDN_WORKLOADS["gdn_layer_bf16"]
    inp = make_gdn_inputs(c, seed=3)
    log(f"[gdn o] full size {c}")
    h, vn, fin = _run_h(ssd, c, inp, torch.bfloat16)
    o = _run_o(ssd, c, inp, vn, h, odt=torch.bfloat16)
    assert torch.isfinite(o.float()).all()
    for (bi, hi) in [(0, 0), (6, 9), (7, 15)]:
        sub = {k: inp[k][bi:bi + 1, :, hi:hi + 1] for k in ("q", "k", "g")}
        ref = oracle.gdn_chunk_fwd_o(sub["q"], sub["k"],
                                     _np(vn[bi:bi + 1, :, hi:hi + 1]).astype(np.float64),
                                     _np(h[bi:bi + 1, hi:hi + 1]).astype(np.float64), sub["g"])
        assert_close(_np(o[bi, :, hi]), ref[0, :, 0], "bf16", f"o[{bi},{hi}]", y_bf16=True)
