"""Mamba-2 SSD chunked forward on AMD Instinct MI355X (gfx950).

A thin Python binding over libssd's C ABI (``include/ssd.h``).  Every step of
the computation runs in the library's HIP kernels; this module only checks
tensor shapes/dtypes, builds the dims struct and passes device pointers and
the current HIP stream.  PyTorch supplies device memory and streams.

Entry points (same names as the C ABI):
  ssd_chunk_cumsum, ssd_fwd_pass_state, ssd_chunk_state, ssd_state_passing,
  ssd_compute_out, ssd_state_and_out, ssd_forward, ssd_forward_noalloc,
  ssd_decode_step, ssd_causal_conv1d, ssd_gdn_chunk_fwd_h, ssd_gdn_chunk_fwd_o
and the allocating convenience wrapper ``forward``.

Importing fails loudly (ImportError) when libssd.so has not been built:
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ssd.h")

SSD_OK = 0
SSD_ERR_INVALID_ARGUMENT = 1
SSD_ERR_UNSUPPORTED = 2
SSD_ERR_WORKSPACE = 3
SSD_ERR_HIP = 4
SSD_F32 = 0
SSD_BF16 = 1


class SsdDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk_size", ctypes.c_int64)]


class GdnDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("dk", ctypes.c_int64),
                ("dv", ctypes.c_int64), ("chunk_size", ctypes.c_int64)]


class SsdError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"libssd.so not found at {LIB_PATH}; build it with "
            "`python mamba_ssd_chunked_fwd_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    dims = ctypes.POINTER(SsdDims)
    lib.ssd_status_string.argtypes = [i]
    lib.ssd_status_string.restype = ctypes.c_char_p
    lib.ssd_forward_workspace_bytes.argtypes = [dims]
    lib.ssd_forward_workspace_bytes.restype = sz
    lib.ssd_chunk_cumsum.argtypes = [vp, vp, vp, vp, dims, vp]
    lib.ssd_chunk_cumsum.restype = i
    lib.ssd_fwd_pass_state.argtypes = [vp] * 7 + [i, dims, vp]
    lib.ssd_fwd_pass_state.restype = i
    lib.ssd_chunk_state.argtypes = [vp] * 6 + [i, dims, vp]
    lib.ssd_chunk_state.restype = i
    lib.ssd_state_passing.argtypes = [vp] * 4 + [dims, vp]
    lib.ssd_state_passing.restype = i
    lib.ssd_compute_out.argtypes = [vp] * 8 + [i, i, dims, vp]
    lib.ssd_compute_out.restype = i
    lib.ssd_state_and_out.argtypes = [vp] * 10 + [i, i, dims, vp]
    lib.ssd_state_and_out.restype = i
    lib.ssd_forward.argtypes = [vp] * 11 + [sz, i, i, dims, vp]
    lib.ssd_forward.restype = i
    lib.ssd_forward_noalloc.argtypes = [vp] * 10 + [i, i, dims, vp]
    lib.ssd_forward_noalloc.restype = i
    lib.ssd_decode_step.argtypes = [vp] * 8 + [i, i, dims, vp]
    lib.ssd_decode_step.restype = i
    i64 = ctypes.c_int64
    gdims = ctypes.POINTER(GdnDims)
    lib.ssd_gdn_chunk_fwd_h.argtypes = [vp] * 8 + [i, i, gdims, vp]
    lib.ssd_gdn_chunk_fwd_h.restype = i
    lib.ssd_gdn_chunk_fwd_o.argtypes = [vp] * 6 + [ctypes.c_float, i, i, i, gdims, vp]
    lib.ssd_gdn_chunk_fwd_o.restype = i
    lib.ssd_causal_conv1d.argtypes = [vp] * 4 + [i64] * 4 + [i, i, vp]
    lib.ssd_causal_conv1d.restype = i
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    """The loaded libssd handle."""
    return _lib


def header_functions() -> list:
    """Names of the functions include/ssd.h declares."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                      r"(ssd_[a-z0-9_]+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    return _lib.ssd_status_string(int(status)).decode()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return SSD_F32
    if t == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"unsupported dtype {t}; expected float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: Optional[torch.Tensor], name: str, shape, dtypes,
           device=None, optional=False) -> None:
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % 16:
        raise ValueError(f"{name} must start on a 16-byte boundary (a slice of a "
                         f"larger tensor may not; pass a copy)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected "
                         f"{tuple(shape)}")


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def make_dims(x: torch.Tensor, B: torch.Tensor, chunk_size: int) -> SsdDims:
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [batch, seqlen, nheads, headdim] and B "
                         "[batch, seqlen, ngroups, dstate]")
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return SsdDims(b, L, H, P, N, G, int(chunk_size))


def nchunks(d: SsdDims) -> int:
    return -(-d.seqlen // d.chunk_size)


def workspace_bytes(d: SsdDims) -> int:
    return int(_lib.ssd_forward_workspace_bytes(ctypes.byref(d)))


def _raise(st: int, where: str) -> None:
    if st != SSD_OK:
        raise SsdError(st, where)


# ------------------------------------------------------------- C-ABI entries
def ssd_chunk_cumsum(dt: torch.Tensor, A: torch.Tensor, g: torch.Tensor,
                     dt_t: torch.Tensor, chunk_size: int) -> None:
    """Stage 1: g [b, H, L] = log2(e) * per-chunk inclusive cumsum of A dt,
    and dt_t [b, H, L], dt transposed to head-major."""
    if dt.dim() != 3:
        raise ValueError("dt must be [batch, seqlen, nheads]")
    b, L, H = dt.shape
    f32 = (torch.float32,)
    _check(dt, "dt", None, f32)
    _check(A, "A", (H,), f32, dt.device)
    _check(g, "g", (b, H, L), f32, dt.device)
    _check(dt_t, "dt_t", (b, H, L), f32, dt.device)
    # stage 1 reads only batch, seqlen, nheads and chunk_size
    d = SsdDims(b, L, H, 64, 64, 1, int(chunk_size))
    _raise(_lib.ssd_chunk_cumsum(_ptr(dt), _ptr(A), _ptr(g), _ptr(dt_t),
                                 ctypes.byref(d), _stream(dt.device)),
           "ssd_chunk_cumsum")


def ssd_fwd_pass_state(x: torch.Tensor, B: torch.Tensor, dt_t: torch.Tensor,
                       g: torch.Tensor, init_state: Optional[torch.Tensor],
                       states: torch.Tensor,
                       final_state: Optional[torch.Tensor],
                       chunk_size: int) -> None:
    """Stage 2: per-chunk starting states [b, H, nc, P, N] and the final state."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    _check(B, "B", (d.batch, d.seqlen, d.ngroups, d.dstate), (x.dtype,), dev)
    _check(dt_t, "dt_t", (d.batch, d.nheads, d.seqlen), f32, dev)
    _check(g, "g", (d.batch, d.nheads, d.seqlen), f32, dev)
    st_shape = (d.batch, d.nheads, d.headdim, d.dstate)
    _check(init_state, "init_state", st_shape, f32, dev, optional=True)
    _check(states, "states", (d.batch, d.nheads, nchunks(d), d.headdim,
                              d.dstate), f32, dev)
    _check(final_state, "final_state", st_shape, f32, dev, optional=True)
    _raise(_lib.ssd_fwd_pass_state(
        _ptr(x), _ptr(B), _ptr(dt_t), _ptr(g), _ptr(init_state), _ptr(states),
        _ptr(final_state), _dtype_code(x.dtype), ctypes.byref(d),
        _stream(dev)), "ssd_fwd_pass_state")


def ssd_chunk_state(x: torch.Tensor, B: torch.Tensor, dt_t: torch.Tensor,
                    g: torch.Tensor, states: torch.Tensor,
                    final_state: Optional[torch.Tensor], chunk_size: int) -> None:
    """Every chunk's zero-state contribution P_c into states[:, :, c+1]
    (P_{nc-1} into final_state); states[:, :, 0] is left as it is."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    b, L, H, P, N, nc = d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, nchunks(d)
    f32 = (torch.float32,)
    _check(x, "x", None, (torch.float32, torch.bfloat16))
    _check(B, "B", (b, L, d.ngroups, N), (x.dtype,), dev)
    _check(dt_t, "dt_t", (b, H, L), f32, dev)
    _check(g, "g", (b, H, L), f32, dev)
    _check(states, "states", (b, H, nc, P, N), f32, dev)
    _check(final_state, "final_state", (b, H, P, N), f32, dev, optional=True)
    _raise(_lib.ssd_chunk_state(
        _ptr(x), _ptr(B), _ptr(dt_t), _ptr(g), _ptr(states), _ptr(final_state),
        _dtype_code(x.dtype), ctypes.byref(d), _stream(dev)), "ssd_chunk_state")


def ssd_state_passing(g: torch.Tensor, init_state: Optional[torch.Tensor],
                      states: torch.Tensor, final_state: Optional[torch.Tensor],
                      chunk_size: int) -> None:
    """In place: the chunk contributions left by ssd_chunk_state become the
    per-chunk starting states (and the final state)."""
    if states.dim() != 5:
        raise ValueError("states must be [batch, nheads, nchunks, headdim, dstate]")
    b, H, nc, P, N = states.shape
    L = g.shape[2] if g.dim() == 3 else -1
    dev = states.device
    f32 = (torch.float32,)
    _check(g, "g", (b, H, L), f32, dev)
    if -(-L // chunk_size) != nc:
        raise ValueError(f"states has {nc} chunks; g's {L} tokens make "
                         f"{-(-L // chunk_size)} chunks of {chunk_size}")
    _check(states, "states", None, f32, dev)
    _check(init_state, "init_state", (b, H, P, N), f32, dev, optional=True)
    _check(final_state, "final_state", (b, H, P, N), f32, dev, optional=True)
    d = SsdDims(b, L, H, P, N, 1, chunk_size)
    _raise(_lib.ssd_state_passing(
        _ptr(g), _ptr(init_state), _ptr(states), _ptr(final_state), ctypes.byref(d),
        _stream(dev)), "ssd_state_passing")


def ssd_compute_out(x: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                    dt_t: torch.Tensor, g: torch.Tensor, states: torch.Tensor,
                    D: torch.Tensor, y: torch.Tensor, chunk_size: int) -> None:
    """Stage 3: y [b, L, H, P] from the per-chunk starting states."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    bc = (d.batch, d.seqlen, d.ngroups, d.dstate)
    _check(B, "B", bc, (x.dtype,), dev)
    _check(C, "C", bc, (x.dtype,), dev)
    _check(dt_t, "dt_t", (d.batch, d.nheads, d.seqlen), f32, dev)
    _check(g, "g", (d.batch, d.nheads, d.seqlen), f32, dev)
    _check(states, "states", (d.batch, d.nheads, nchunks(d), d.headdim,
                              d.dstate), f32, dev)
    _check(D, "D", (d.nheads,), f32, dev)
    _check(y, "y", tuple(x.shape), ins, dev)
    _raise(_lib.ssd_compute_out(
        _ptr(x), _ptr(B), _ptr(C), _ptr(dt_t), _ptr(g), _ptr(states), _ptr(D),
        _ptr(y), _dtype_code(x.dtype), _dtype_code(y.dtype), ctypes.byref(d),
        _stream(dev)), "ssd_compute_out")


def ssd_state_and_out(x: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                      dt_t: torch.Tensor, g: torch.Tensor, D: torch.Tensor,
                      init_state: Optional[torch.Tensor], y: torch.Tensor,
                      states: torch.Tensor, final_state: Optional[torch.Tensor],
                      chunk_size: int) -> None:
    """Stages 2 and 3 in one call (the fused single pass where it applies):
    states, final_state and y from stage 1's g and dt_t."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    bc = (d.batch, d.seqlen, d.ngroups, d.dstate)
    _check(B, "B", bc, (x.dtype,), dev)
    _check(C, "C", bc, (x.dtype,), dev)
    _check(dt_t, "dt_t", (d.batch, d.nheads, d.seqlen), f32, dev)
    _check(g, "g", (d.batch, d.nheads, d.seqlen), f32, dev)
    _check(D, "D", (d.nheads,), f32, dev)
    st_shape = (d.batch, d.nheads, d.headdim, d.dstate)
    _check(init_state, "init_state", st_shape, f32, dev, optional=True)
    _check(y, "y", tuple(x.shape), ins, dev)
    _check(states, "states", (d.batch, d.nheads, nchunks(d), d.headdim,
                              d.dstate), f32, dev)
    _check(final_state, "final_state", st_shape, f32, dev, optional=True)
    _raise(_lib.ssd_state_and_out(
        _ptr(x), _ptr(B), _ptr(C), _ptr(dt_t), _ptr(g), _ptr(D), _ptr(init_state),
        _ptr(y), _ptr(states), _ptr(final_state), _dtype_code(x.dtype),
        _dtype_code(y.dtype), ctypes.byref(d), _stream(dev)), "ssd_state_and_out")


def ssd_forward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                B: torch.Tensor, C: torch.Tensor, D: torch.Tensor,
                init_state: Optional[torch.Tensor], y: torch.Tensor,
                states: torch.Tensor, final_state: Optional[torch.Tensor],
                workspace: torch.Tensor, chunk_size: int) -> None:
    """All three stages on the current stream; g and dt_t live in
    ``workspace`` (``workspace_bytes`` bytes)."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    bc = (d.batch, d.seqlen, d.ngroups, d.dstate)
    _check(B, "B", bc, (x.dtype,), dev)
    _check(C, "C", bc, (x.dtype,), dev)
    _check(dt, "dt", (d.batch, d.seqlen, d.nheads), f32, dev)
    _check(A, "A", (d.nheads,), f32, dev)
    _check(D, "D", (d.nheads,), f32, dev)
    st_shape = (d.batch, d.nheads, d.headdim, d.dstate)
    _check(init_state, "init_state", st_shape, f32, dev, optional=True)
    _check(y, "y", tuple(x.shape), ins, dev)
    _check(states, "states", (d.batch, d.nheads, nchunks(d), d.headdim,
                              d.dstate), f32, dev)
    _check(final_state, "final_state", st_shape, f32, dev, optional=True)
    _check(workspace, "workspace", None, (torch.uint8, torch.float32), dev)
    nbytes = workspace.numel() * workspace.element_size()
    _raise(_lib.ssd_forward(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(init_state), _ptr(y), _ptr(states), _ptr(final_state),
        _ptr(workspace), nbytes, _dtype_code(x.dtype), _dtype_code(y.dtype),
        ctypes.byref(d), _stream(dev)), "ssd_forward")


NOALLOC_SCRATCH_BYTES = 32 << 20


def ssd_forward_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                        B: torch.Tensor, C: torch.Tensor, D: torch.Tensor,
                        init_state: Optional[torch.Tensor], y: torch.Tensor,
                        states: torch.Tensor, final_state: Optional[torch.Tensor],
                        chunk_size: int) -> None:
    """``ssd_forward`` without a workspace: g and dt_t live in the library's
    per-GPU scratch array (NOALLOC_SCRATCH_BYTES), so the call allocates
    nothing.  Calls that overlap in time on one GPU race on that array."""
    d = make_dims(x, B, chunk_size)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    bc = (d.batch, d.seqlen, d.ngroups, d.dstate)
    _check(B, "B", bc, (x.dtype,), dev)
    _check(C, "C", bc, (x.dtype,), dev)
    _check(dt, "dt", (d.batch, d.seqlen, d.nheads), f32, dev)
    _check(A, "A", (d.nheads,), f32, dev)
    _check(D, "D", (d.nheads,), f32, dev)
    st_shape = (d.batch, d.nheads, d.headdim, d.dstate)
    _check(init_state, "init_state", st_shape, f32, dev, optional=True)
    _check(y, "y", tuple(x.shape), ins, dev)
    _check(states, "states", (d.batch, d.nheads, nchunks(d), d.headdim,
                              d.dstate), f32, dev)
    _check(final_state, "final_state", st_shape, f32, dev, optional=True)
    _raise(_lib.ssd_forward_noalloc(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(init_state), _ptr(y), _ptr(states), _ptr(final_state),
        _dtype_code(x.dtype), _dtype_code(y.dtype), ctypes.byref(d), _stream(dev)),
        "ssd_forward_noalloc")


def ssd_decode_step(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
                    B: torch.Tensor, C: torch.Tensor, D: torch.Tensor,
                    state: torch.Tensor, y: torch.Tensor) -> None:
    """One token for every (batch, head): ``state`` [b, H, P, N] fp32 is
    updated in place and ``y`` [b, H, P] written.  x [b, H, P], dt [b, H],
    B, C [b, G, N]."""
    if x.dim() != 3 or B.dim() != 3:
        raise ValueError("x must be [batch, nheads, headdim] and B "
                         "[batch, ngroups, dstate]")
    b, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    d = SsdDims(b, 1, H, P, N, G, 64)
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    _check(B, "B", (b, G, N), (x.dtype,), dev)
    _check(C, "C", (b, G, N), (x.dtype,), dev)
    _check(dt, "dt", (b, H), f32, dev)
    _check(A, "A", (H,), f32, dev)
    _check(D, "D", (H,), f32, dev)
    _check(state, "state", (b, H, P, N), f32, dev)
    _check(y, "y", (b, H, P), ins, dev)
    _raise(_lib.ssd_decode_step(
        _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D), _ptr(state),
        _ptr(y), _dtype_code(x.dtype), _dtype_code(y.dtype), ctypes.byref(d),
        _stream(dev)), "ssd_decode_step")


def ssd_gdn_chunk_fwd_h(k: torch.Tensor, w: torch.Tensor, u: torch.Tensor,
                        g: torch.Tensor, h0: Optional[torch.Tensor],
                        h: torch.Tensor, v_new: torch.Tensor,
                        final_state: Optional[torch.Tensor],
                        chunk_size: int = 64) -> None:
    """Gated DeltaNet state pass: k, w [b, L, H, K] and u [b, L, H, V] (bf16),
    g [b, L, H] fp32, h0 [b, H, K, V] fp32 or None; writes h [b, H, nt, K, V]
    fp32, v_new [b, L, H, V] (fp32 or bf16) and final_state (or None)."""
    if k.dim() != 4 or u.dim() != 4:
        raise ValueError("k must be [batch, seqlen, nheads, dk] and u "
                         "[batch, seqlen, nheads, dv]")
    b, L, H, K = k.shape
    V = u.shape[3]
    nt = -(-L // chunk_size)
    dev = k.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(k, "k", None, ins)
    _check(w, "w", (b, L, H, K), (k.dtype,), dev)
    _check(u, "u", (b, L, H, V), (k.dtype,), dev)
    _check(g, "g", (b, L, H), f32, dev)
    _check(h0, "h0", (b, H, K, V), f32, dev, optional=True)
    _check(h, "h", (b, H, nt, K, V), f32, dev)
    _check(v_new, "v_new", (b, L, H, V), ins, dev)
    _check(final_state, "final_state", (b, H, K, V), f32, dev, optional=True)
    d = GdnDims(b, L, H, K, V, chunk_size)
    _raise(_lib.ssd_gdn_chunk_fwd_h(
        _ptr(k), _ptr(w), _ptr(u), _ptr(g), _ptr(h0), _ptr(h), _ptr(v_new),
        _ptr(final_state), _dtype_code(k.dtype), _dtype_code(v_new.dtype),
        ctypes.byref(d), _stream(dev)), "ssd_gdn_chunk_fwd_h")


def ssd_gdn_chunk_fwd_o(q: torch.Tensor, k: torch.Tensor, v_new: torch.Tensor,
                        h: torch.Tensor, g: torch.Tensor, o: torch.Tensor,
                        scale: float = 1.0, chunk_size: int = 64) -> None:
    """Gated DeltaNet output: q, k [b, L, H, K] bf16; v_new [b, L, H, V] bf16;
    h [b, H, nt, K, V] fp32; g [b, L, H] fp32; writes o [b, L, H, V]
    (fp32 or bf16)."""
    if q.dim() != 4 or v_new.dim() != 4:
        raise ValueError("q must be [batch, seqlen, nheads, dk] and v_new "
                         "[batch, seqlen, nheads, dv]")
    b, L, H, K = q.shape
    V = v_new.shape[3]
    nt = -(-L // chunk_size)
    dev = q.device
    ins = (torch.float32, torch.bfloat16)
    _check(q, "q", None, ins)
    _check(k, "k", (b, L, H, K), (q.dtype,), dev)
    _check(v_new, "v_new", (b, L, H, V), ins, dev)
    _check(h, "h", (b, H, nt, K, V), (torch.float32,), dev)
    _check(g, "g", (b, L, H), (torch.float32,), dev)
    _check(o, "o", (b, L, H, V), ins, dev)
    d = GdnDims(b, L, H, K, V, chunk_size)
    _raise(_lib.ssd_gdn_chunk_fwd_o(
        _ptr(q), _ptr(k), _ptr(v_new), _ptr(h), _ptr(g), _ptr(o),
        ctypes.c_float(scale), _dtype_code(q.dtype), _dtype_code(v_new.dtype),
        _dtype_code(o.dtype), ctypes.byref(d), _stream(dev)), "ssd_gdn_chunk_fwd_o")


def ssd_causal_conv1d(x: torch.Tensor, weight: torch.Tensor,
                      bias: Optional[torch.Tensor], out: torch.Tensor) -> None:
    """Causal depthwise conv1d: x [batch, dim, seqlen] (fp32 or bf16),
    weight [dim, width] fp32, bias [dim] fp32 or None; writes ``out``
    [batch, dim, seqlen] (fp32 or bf16)."""
    if x.dim() != 3 or weight.dim() != 2:
        raise ValueError("x must be [batch, dim, seqlen] and weight "
                         "[dim, width]")
    b, dim, L = x.shape
    W = weight.shape[1]
    dev = x.device
    ins = (torch.float32, torch.bfloat16)
    f32 = (torch.float32,)
    _check(x, "x", None, ins)
    _check(weight, "weight", (dim, W), f32, dev)
    _check(bias, "bias", (dim,), f32, dev, optional=True)
    _check(out, "out", (b, dim, L), ins, dev)
    _raise(_lib.ssd_causal_conv1d(
        _ptr(x), _ptr(weight), _ptr(bias), _ptr(out), b, dim, L, W,
        _dtype_code(x.dtype), _dtype_code(out.dtype), _stream(dev)),
        "ssd_causal_conv1d")


# ------------------------------------------------------------ convenience
def forward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
            B: torch.Tensor, C: torch.Tensor, D: torch.Tensor,
            init_state: Optional[torch.Tensor] = None, chunk_size: int = 64,
            y_dtype: torch.dtype = torch.float32
            ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Allocate outputs with torch.empty and run ``ssd_forward``.

    Returns (y [b, L, H, P] in y_dtype, states [b, H, nc, P, N] fp32,
    final_state [b, H, P, N] fp32).
    """
    d = make_dims(x, B, chunk_size)
    dev = x.device
    y = torch.empty(tuple(x.shape), dtype=y_dtype, device=dev)
    states = torch.empty((d.batch, d.nheads, nchunks(d), d.headdim, d.dstate),
                         dtype=torch.float32, device=dev)
    final = torch.empty((d.batch, d.nheads, d.headdim, d.dstate),
                        dtype=torch.float32, device=dev)
    # invalid or unsupported dims report 0 bytes; ssd_forward then returns the
    # precise status before touching the (minimal) workspace
    nbytes = max(workspace_bytes(d), 16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    ssd_forward(x, dt, A, B, C, D, init_state, y, states, final, ws,
                chunk_size)
    return y, states, final
