"""The seeded input generator: determinism, shapes, domains, bf16 rounding."""
import numpy as np
import pytest

from ssd_workloads import WORKLOADS, make_inputs, round_to_bf16, small_variant


def test_round_to_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 100,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875,
                                  3.0e38, -3.0e38, 1e-40], np.float32)])
    ours = round_to_bf16(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name", ["tiny_fp32", "small_bf16", "wide_fp32"])
def test_shapes_domains_and_determinism(name):
    w = WORKLOADS[name]
    if w.batch * w.seqlen * w.nheads > 4_000_000:
        w = small_variant(w, batch=2, seqlen=256)
    a = make_inputs(w)
    b = make_inputs(w)
    for k in a:
        if a[k] is None:
            assert b[k] is None
        else:
            assert np.array_equal(a[k], b[k])
    B_, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    assert a["x"].shape == (B_, L, H, P)
    assert a["B"].shape == a["C"].shape == (B_, L, G, N)
    assert a["dt"].shape == (B_, L, H)
    assert a["A"].shape == a["D"].shape == (H,)
    assert np.all(a["dt"] > 0) and np.all(a["A"] < 0)
    if w.dtype == "bf16":
        for k in ("x", "B", "C"):
            assert np.all((a[k].view(np.uint32) & 0xFFFF) == 0)
    c = make_inputs(w, seed=123)
    assert not np.array_equal(a["x"], c["x"])


def test_named_workloads_match_their_description():
    w = WORKLOADS
    assert (w["small_bf16"].batch, w["small_bf16"].seqlen, w["small_bf16"].nheads,
            w["small_bf16"].dstate, w["small_bf16"].chunk_size) == (4, 2048, 24, 128, 64)
    assert (w["large_bf16"].batch, w["large_bf16"].seqlen, w["large_bf16"].nheads,
            w["large_bf16"].chunk_size) == (2, 8192, 80, 256)
    assert (w["long_bf16"].seqlen, w["long_bf16"].nheads,
            w["long_bf16"].chunk_size, w["long_bf16"].init_std) == (65536, 32, 128, 0.1)
    assert (w["wide_fp32"].batch, w["wide_fp32"].nheads, w["wide_fp32"].ngroups,
            w["wide_fp32"].dstate) == (64, 48, 8, 64)
    for v in w.values():
        assert v.headdim == 64 and v.nheads % v.ngroups == 0


def test_init_state_distribution():
    w = small_variant(WORKLOADS["long_bf16"], seqlen=128, nheads=4)
    a = make_inputs(w)
    s = a["init_state"]
    assert s.shape == (1, 4, 64, 128) and s.dtype == np.float32
    assert 0.09 < s.std() < 0.11
