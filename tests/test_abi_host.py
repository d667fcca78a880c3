"""Host-side checks of the C ABI (no GPU needed).

Every call below fails argument validation, which the library performs on the
host before any HIP call, so nothing is launched and no pointer is touched.
The calls pass fake device addresses, so the module refuses to run where a
GPU is visible: a mistaken case there could launch a kernel on them.
"""
import ctypes
import subprocess

import pytest

try:
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-only validation tests use fake device pointers; "
                    "not run where a GPU is visible", allow_module_level=True)
except ImportError:  # pragma: no cover
    pass

import mamba_ssd_chunked_fwd_amd as ssd
from mamba_ssd_chunked_fwd_amd import SsdDims

OK, INV, UNS, WS = (ssd.SSD_OK, ssd.SSD_ERR_INVALID_ARGUMENT,
                    ssd.SSD_ERR_UNSUPPORTED, ssd.SSD_ERR_WORKSPACE)
lib = ssd.library()
FAKE = ctypes.c_void_p(0x7F0000000000)       # 16-byte aligned, never used
MISALIGNED = ctypes.c_void_p(0x7F0000000004)


def dims(**kw):
    base = dict(batch=2, seqlen=256, nheads=4, headdim=64, dstate=128,
                ngroups=2, chunk_size=64)
    base.update(kw)
    return SsdDims(**base)


def test_every_declared_function_is_exported():
    names = ssd.header_functions()
    assert set(names) == {"ssd_status_string", "ssd_forward_workspace_bytes",
                          "ssd_chunk_cumsum", "ssd_fwd_pass_state",
                          "ssd_compute_out", "ssd_forward", "ssd_decode_step",
                          "ssd_causal_conv1d", "ssd_gdn_chunk_fwd_h",
                          "ssd_gdn_chunk_fwd_o", "ssd_chunk_state",
                          "ssd_state_passing", "ssd_forward_noalloc",
                          "ssd_state_and_out"}
    out = subprocess.run(["nm", "-D", "--defined-only", ssd.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)


def test_status_strings():
    assert ssd.status_string(OK) == "SSD_OK"
    assert ssd.status_string(INV) == "SSD_ERR_INVALID_ARGUMENT"
    assert ssd.status_string(UNS) == "SSD_ERR_UNSUPPORTED"
    assert ssd.status_string(WS) == "SSD_ERR_WORKSPACE"
    assert ssd.status_string(ssd.SSD_ERR_HIP) == "SSD_ERR_HIP"
    assert ssd.status_string(99) == "SSD_ERR_UNKNOWN"


def test_workspace_bytes():
    d = dims()
    assert ssd.workspace_bytes(d) == 8 * 2 * 4 * 256
    assert ssd.workspace_bytes(dims(seqlen=1000, chunk_size=256)) == 8 * 2 * 4 * 1000
    assert ssd.workspace_bytes(dims(headdim=32)) == 0
    assert ssd.workspace_bytes(dims(nheads=5)) == 0
    assert lib.ssd_forward_workspace_bytes(None) == 0


def _fwd(d, **over):
    need = ssd.workspace_bytes(d) if d is not None else 0
    args = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=FAKE, init=None,
                y=FAKE, states=FAKE, final=None, ws=FAKE,
                wsb=need if need else 1 << 20,
                ind=ssd.SSD_BF16, yd=ssd.SSD_F32)
    args.update(over)
    return lib.ssd_forward(args["x"], args["dt"], args["A"], args["B"],
                           args["C"], args["D"], args["init"], args["y"],
                           args["states"], args["final"], args["ws"],
                           args["wsb"], args["ind"], args["yd"],
                           ctypes.byref(d) if d is not None else None, None)


@pytest.mark.parametrize("field,value,expect", [
    ("batch", 0, INV), ("seqlen", 0, INV), ("nheads", -1, INV),
    ("ngroups", 3, INV),                     # 4 % 3 != 0
    ("headdim", 32, UNS), ("headdim", 128, UNS),
    ("dstate", 256, UNS), ("dstate", 16, UNS),
    ("chunk_size", 32, UNS), ("chunk_size", 100, UNS),
    ("seqlen", 1 << 40, INV),
    ("seqlen", 1 << 22, UNS),                # per-sequence extent >= 2 GiB
])
def test_forward_rejects_bad_dims(field, value, expect):
    assert _fwd(dims(**{field: value})) == expect


def test_forward_rejects_null_and_misaligned_pointers():
    d = dims()
    assert _fwd(None) == INV
    for name in ("x", "dt", "A", "B", "C", "D", "y", "states"):
        assert _fwd(d, **{name: None}) == INV, name
        assert _fwd(d, **{name: MISALIGNED}) == INV, name
    assert _fwd(d, init=MISALIGNED) == INV
    assert _fwd(d, final=MISALIGNED) == INV
    assert _fwd(d, ind=2) == INV
    assert _fwd(d, yd=-1) == INV


def test_forward_rejects_small_workspace():
    d = dims()
    need = ssd.workspace_bytes(d)
    assert _fwd(d, wsb=need - 1) == WS
    assert _fwd(d, ws=None) == WS
    assert _fwd(d, ws=MISALIGNED) == WS


def test_decode_step_validates():
    d = dims()
    call = lambda dd, **o: lib.ssd_decode_step(
        o.get("x", FAKE), o.get("dt", FAKE), o.get("A", FAKE), o.get("B", FAKE),
        o.get("C", FAKE), o.get("D", FAKE), o.get("state", FAKE), o.get("y", FAKE),
        o.get("ind", ssd.SSD_BF16), o.get("yd", ssd.SSD_F32),
        ctypes.byref(dd) if dd is not None else None, None)
    assert call(None) == INV
    for name in ("x", "dt", "A", "B", "C", "D", "state", "y"):
        assert call(d, **{name: None}) == INV, name
        assert call(d, **{name: MISALIGNED}) == INV, name
    assert call(d, ind=3) == INV
    assert call(dims(dstate=96)) == UNS
    assert call(dims(headdim=128)) == UNS
    assert call(dims(nheads=5)) == INV          # 5 heads, 2 groups


def test_causal_conv1d_validates():
    def call(b=2, d=8, L=64, W=4, **o):
        return lib.ssd_causal_conv1d(
            o.get("x", FAKE), o.get("w", FAKE), o.get("bias", FAKE),
            o.get("out", FAKE), b, d, L, W, o.get("xd", ssd.SSD_BF16),
            o.get("od", ssd.SSD_BF16), None)
    for name in ("x", "w", "out"):
        assert call(**{name: None}) == INV, name
        assert call(**{name: MISALIGNED}) == INV, name
    assert call(bias=MISALIGNED) == INV
    for kw in (dict(b=0), dict(d=0), dict(L=0), dict(W=0), dict(L=-5)):
        assert call(**kw) == INV, kw
    assert call(xd=2) == INV
    assert call(od=-1) == INV
    assert call(W=5) == UNS
    assert call(L=1 << 29) == UNS
    assert call(b=1 << 30, d=1 << 12, L=1 << 12) == UNS


def test_two_level_entry_points_validate():
    d = dims()
    cs = lambda dd, **o: lib.ssd_chunk_state(
        o.get("x", FAKE), o.get("B", FAKE), o.get("dtt", FAKE), o.get("g", FAKE),
        o.get("st", FAKE), o.get("fin", None), o.get("ind", ssd.SSD_BF16),
        ctypes.byref(dd) if dd is not None else None, None)
    sp = lambda dd, **o: lib.ssd_state_passing(
        o.get("g", FAKE), o.get("init", None), o.get("st", FAKE), o.get("fin", None),
        ctypes.byref(dd) if dd is not None else None, None)
    assert cs(None) == INV and sp(None) == INV
    for name in ("x", "B", "dtt", "g", "st"):
        assert cs(d, **{name: None}) == INV, name
        assert cs(d, **{name: MISALIGNED}) == INV, name
    assert cs(d, fin=MISALIGNED) == INV and cs(d, ind=9) == INV
    assert cs(dims(dstate=96)) == UNS and sp(dims(dstate=96)) == UNS
    for name in ("g", "st"):
        assert sp(d, **{name: None}) == INV, name
    assert sp(d, init=MISALIGNED) == INV and sp(d, fin=MISALIGNED) == INV
    # final_state carries P_{nc-1} between the two calls: it may not overlap
    # the initial state (whole or partial overlap)
    assert sp(d, init=FAKE, fin=FAKE) == INV
    assert sp(d, init=ctypes.c_void_p(FAKE.value + 4096), fin=FAKE) == INV
    assert sp(d, init=FAKE, fin=ctypes.c_void_p(FAKE.value + 16)) == INV


def test_gdn_entry_points_validate():
    GD = ssd.GdnDims

    def gd(**kw):
        base = dict(batch=2, seqlen=256, nheads=4, dk=128, dv=128, chunk_size=64)
        base.update(kw)
        return GD(**base)

    def fh(d, **o):
        return lib.ssd_gdn_chunk_fwd_h(
            o.get("k", FAKE), o.get("w", FAKE), o.get("u", FAKE), o.get("g", FAKE),
            o.get("h0", None), o.get("h", FAKE), o.get("vn", FAKE), o.get("fin", None),
            o.get("ind", ssd.SSD_BF16), o.get("vd", ssd.SSD_BF16),
            ctypes.byref(d) if d is not None else None, None)

    def fo(d, **o):
        return lib.ssd_gdn_chunk_fwd_o(
            o.get("q", FAKE), o.get("k", FAKE), o.get("vn", FAKE), o.get("h", FAKE),
            o.get("g", FAKE), o.get("o", FAKE), ctypes.c_float(1.0),
            o.get("ind", ssd.SSD_BF16), o.get("vd", ssd.SSD_BF16), o.get("od", ssd.SSD_F32),
            ctypes.byref(d) if d is not None else None, None)

    d = gd()
    assert fh(None) == INV and fo(None) == INV
    for name in ("k", "w", "u", "g", "h", "vn"):
        assert fh(d, **{name: None}) == INV, name
        assert fh(d, **{name: MISALIGNED}) == INV, name
    assert fh(d, h0=MISALIGNED) == INV and fh(d, fin=MISALIGNED) == INV
    for name in ("q", "k", "vn", "h", "g", "o"):
        assert fo(d, **{name: None}) == INV, name
    assert fh(d, ind=7) == INV and fo(d, od=7) == INV
    assert fh(d, ind=ssd.SSD_F32) == UNS          # fp32 inputs are not built
    assert fo(d, vd=ssd.SSD_F32) == UNS           # fp32 v_new is not read
    assert fh(gd(dk=96)) == UNS and fo(gd(dv=32)) == UNS
    assert fh(gd(chunk_size=128)) == UNS
    assert fh(gd(seqlen=0)) == INV and fo(gd(nheads=0)) == INV
    assert fh(gd(seqlen=1 << 20, nheads=1024)) == UNS


def test_stage_entry_points_validate():
    d = dims()
    assert lib.ssd_chunk_cumsum(None, FAKE, FAKE, FAKE, ctypes.byref(d), None) == INV
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, FAKE, None, ctypes.byref(d), None) == INV
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, FAKE, FAKE, None, None) == INV
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, FAKE, FAKE,
                                ctypes.byref(dims(chunk_size=48)), None) == UNS
    # stage 1 ignores P, N and G
    assert lib.ssd_chunk_cumsum(FAKE, FAKE, MISALIGNED, FAKE,
                                ctypes.byref(dims(headdim=7)), None) == INV
    assert lib.ssd_fwd_pass_state(FAKE, FAKE, FAKE, FAKE, None, None, None,
                                  ssd.SSD_BF16, ctypes.byref(d), None) == INV
    assert lib.ssd_fwd_pass_state(FAKE, FAKE, FAKE, FAKE, None, FAKE, None, 5,
                                  ctypes.byref(d), None) == INV
    assert lib.ssd_fwd_pass_state(FAKE, FAKE, FAKE, FAKE, None, FAKE, None,
                                  ssd.SSD_F32, ctypes.byref(dims(dstate=96)),
                                  None) == UNS
    assert lib.ssd_compute_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                               ssd.SSD_BF16, ssd.SSD_F32, ctypes.byref(d),
                               None) == INV
    assert lib.ssd_compute_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               ssd.SSD_BF16, 3, ctypes.byref(d), None) == INV
    assert lib.ssd_compute_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               ssd.SSD_BF16, ssd.SSD_F32,
                               ctypes.byref(dims(nheads=6, ngroups=4)), None) == INV
    # stages 2 and 3 in one call: x, B, C, dt_t, g, D, init, y, states, final
    assert lib.ssd_state_and_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None, None,
                                 ssd.SSD_F32, ssd.SSD_F32, ctypes.byref(d), None) == INV
    assert lib.ssd_state_and_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, MISALIGNED, FAKE, FAKE,
                                 None, ssd.SSD_F32, ssd.SSD_F32, ctypes.byref(d), None) == INV
    assert lib.ssd_state_and_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                                 ssd.SSD_F32, 2, ctypes.byref(d), None) == INV
    assert lib.ssd_state_and_out(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None,
                                 ssd.SSD_F32, ssd.SSD_F32,
                                 ctypes.byref(dims(chunk_size=96)), None) == UNS


def test_binding_rejects_cpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 64, 2, 64)
    B = torch.zeros(1, 64, 1, 64)
    with pytest.raises(ValueError):
        ssd.forward(x, torch.zeros(1, 64, 2), torch.zeros(2), B, B,
                    torch.zeros(2), chunk_size=64)


def test_forward_noalloc_validates():
    """Rejections happen on the host before any HIP call; shapes whose g and
    dt_t exceed the per-GPU scratch array get SSD_ERR_WORKSPACE."""
    def call(d, **o):
        return lib.ssd_forward_noalloc(
            o.get("x", FAKE), FAKE, FAKE, FAKE, FAKE, FAKE, o.get("init", None), FAKE, FAKE,
            o.get("fin", None), o.get("ind", ssd.SSD_BF16), ssd.SSD_F32,
            ctypes.byref(d) if d is not None else None, None)
    assert call(None) == INV
    assert call(dims(), x=None) == INV and call(dims(), x=MISALIGNED) == INV
    assert call(dims(), ind=4) == INV
    assert call(dims(headdim=32)) == UNS
    fit = ssd.NOALLOC_SCRATCH_BYTES // 8 // 64          # tokens with 64 heads
    assert ssd.workspace_bytes(dims(batch=1, seqlen=fit, nheads=64, ngroups=1)) == \
        ssd.NOALLOC_SCRATCH_BYTES
    assert call(dims(batch=1, seqlen=fit + 1, nheads=64, ngroups=1)) == WS
    assert call(dims(batch=2, seqlen=fit, nheads=64, ngroups=1)) == WS
