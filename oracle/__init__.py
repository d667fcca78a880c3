"""fp64 CPU oracle for the Mamba-2 SSD chunked forward (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package.  The product path (the HIP library and its Python
binding) never imports, links or runs it, and the two share no code.

The arithmetic lives in ``ssd_oracle.c`` (plain C, fp64, OpenMP over
(batch, head) pairs); this module compiles it with gcc and marshals numpy
arrays.  See the C file's header for what is computed and which passages of
the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Dict, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
# SSD_ORACLE_SANITIZE=1 selects a build with AddressSanitizer and
# UndefinedBehaviorSanitizer (host code only; the process must preload the
# sanitizer runtimes, see sanitizer_env()).
SANITIZE = os.environ.get("SSD_ORACLE_SANITIZE", "") == "1"
_LIB = os.path.join(_HERE, "libssd_oracle_san.so" if SANITIZE else "libssd_oracle.so")
SANITIZER_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                   "-fno-omit-frame-pointer", "-g"]
_lock = threading.Lock()
_lib = None


def build(force: bool = False, sanitize: bool = SANITIZE) -> str:
    """Compile ssd_oracle.c into a shared library with gcc (-O2, OpenMP);
    with `sanitize`, instrumented with ASan and UBSan (-O1)."""
    lib = os.path.join(_HERE, "libssd_oracle_san.so" if sanitize else "libssd_oracle.so")
    if (not force and os.path.exists(lib)
            and os.path.getmtime(lib) >= os.path.getmtime(_SRC)):
        return lib
    tmp = lib + ".tmp%d" % os.getpid()
    opt = ["-O1", *SANITIZER_FLAGS] if sanitize else ["-O2"]
    cmd = ["gcc", *opt, "-fopenmp", "-fPIC", "-shared", "-std=c99",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib)
    return lib


def sanitizer_env(base=None) -> dict:
    """Environment for a process that loads the sanitized oracle: the gcc
    ASan and UBSan runtimes preloaded, leak checking off (the Python
    interpreter itself holds memory until exit)."""
    env = dict(os.environ if base is None else base)
    libs = []
    for name in ("libasan.so", "libubsan.so"):
        p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                           text=True, check=True).stdout.strip()
        libs.append(os.path.realpath(p))
    env["LD_PRELOAD"] = ":".join(libs)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    env["SSD_ORACLE_SANITIZE"] = "1"
    return env


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64, f32p, f64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
            lib.oracle_chunk_cumsum.argtypes = [f32p, f32p, f64p, i64, i64,
                                                i64, i64, ctypes.c_void_p, i64]
            lib.oracle_chunk_cumsum.restype = None
            lib.oracle_forward.argtypes = ([f32p] * 6 + [f64p] * 4 + [i64] * 7
                                           + [ctypes.c_void_p, i64,
                                              ctypes.c_int])
            lib.oracle_forward.restype = None
            lib.oracle_chunk_out.argtypes = ([f32p] * 6 + [f64p, f64p]
                                             + [i64] * 7
                                             + [ctypes.c_void_p, i64,
                                                ctypes.c_int])
            lib.oracle_chunk_out.restype = None
            lib.oracle_causal_conv1d.argtypes = [f32p, f32p, ctypes.c_void_p,
                                                 f64p, i64, i64, i64, i64]
            lib.oracle_causal_conv1d.restype = None
            lib.oracle_gdn_chunk_fwd_h.argtypes = ([f32p] * 4 + [ctypes.c_void_p, f64p, f64p,
                                                   ctypes.c_void_p] + [i64] * 6
                                                  + [ctypes.c_int])
            lib.oracle_gdn_chunk_fwd_h.restype = None
            lib.oracle_gdn_chunk_fwd_o.argtypes = ([f32p, f32p, f64p, f64p, f32p, f64p,
                                                   ctypes.c_double] + [i64] * 6
                                                  + [ctypes.c_int])
            lib.oracle_gdn_chunk_fwd_o.restype = None
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            _lib = lib
    return _lib


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _pairs(pairs, batch, nheads):
    if pairs is None:
        return None, batch * nheads
    p = np.ascontiguousarray(pairs, dtype=np.int64)
    if p.ndim != 1 or (p.size and (p.min() < 0 or p.max() >= batch * nheads)):
        raise ValueError("pairs must be indices b*nheads + h in range")
    return p, int(p.size)


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def chunk_cumsum(dt: np.ndarray, A: np.ndarray, chunk_size: int,
                 pairs: Optional[Sequence[int]] = None) -> np.ndarray:
    """Stage 1: log2(e) * per-chunk inclusive cumsum of A_h * dt.

    dt [b, L, H], A [H] -> g.  With pairs=None returns [b, H, L]; otherwise
    [len(pairs), L] in the order given.
    """
    lib = _load()
    dt, A = _f32(dt), _f32(A)
    b, L, H = dt.shape
    p, npairs = _pairs(pairs, b, H)
    g = np.empty((npairs, L), dtype=np.float64)
    lib.oracle_chunk_cumsum(_ptr(dt), _ptr(A), _ptr(g), b, L, H, chunk_size,
                            _ptr(p), npairs)
    return g.reshape(b, H, L) if pairs is None else g


def forward(x, dt, A, B, C, D, init_state=None, *, chunk_size: int,
            pairs: Optional[Sequence[int]] = None, want_y: bool = True,
            want_states: bool = True, nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Token-by-token recurrence in fp64.

    Returns a dict with
      y      [b, L, H, P]      (pairs=None) or [npairs, L, P]
      states [b, H, nc, P, N]  (pairs=None) or [npairs, nc, P, N]
      final  [b, H, P, N]      (pairs=None) or [npairs, P, N]
    """
    lib = _load()
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    init = (None if init_state is None
            else np.ascontiguousarray(init_state, dtype=np.float64))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = -(-L // chunk_size)
    p, npairs = _pairs(pairs, b, H)
    y = np.empty((npairs, L, P), np.float64) if want_y else None
    st = np.empty((npairs, nc, P, N), np.float64) if want_states else None
    fin = np.empty((npairs, P, N), np.float64)
    lib.oracle_forward(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
                       _ptr(init), _ptr(y), _ptr(st), _ptr(fin), b, L, H, P,
                       N, G, chunk_size, _ptr(p), npairs, nthreads)
    out = {"final": fin}
    if pairs is None:
        out["final"] = fin.reshape(b, H, P, N)
        if want_y:
            out["y"] = y.reshape(b, H, L, P).transpose(0, 2, 1, 3)
        if want_states:
            out["states"] = st.reshape(b, H, nc, P, N)
    else:
        if want_y:
            out["y"] = y
        if want_states:
            out["states"] = st
    return out


def chunk_out(x, dt, A, B, C, D, states, *, chunk_size: int,
              pairs: Optional[Sequence[int]] = None, nthreads: int = 0):
    """Per-chunk outputs, restarting the recurrence from given states.

    states: [b, H, nc, P, N] when pairs=None, else [npairs, nc, P, N]
    (any float dtype; used in fp64).  Returns y in the same convention as
    ``forward``.
    """
    lib = _load()
    x, dt, A, B, C, D = map(_f32, (x, dt, A, B, C, D))
    b, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    nc = -(-L // chunk_size)
    p, npairs = _pairs(pairs, b, H)
    st = np.ascontiguousarray(states, dtype=np.float64).reshape(npairs, nc,
                                                                 P, N)
    y = np.empty((npairs, L, P), np.float64)
    lib.oracle_chunk_out(_ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                         _ptr(D), _ptr(st), _ptr(y), b, L, H, P, N, G,
                         chunk_size, _ptr(p), npairs, nthreads)
    if pairs is None:
        return y.reshape(b, H, L, P).transpose(0, 2, 1, 3)
    return y


def causal_conv1d(x: np.ndarray, weight: np.ndarray,
                  bias: Optional[np.ndarray] = None) -> np.ndarray:
    """Causal depthwise conv1d in fp64: x [batch, dim, seqlen], weight
    [dim, width], bias [dim] or None -> out [batch, dim, seqlen]."""
    lib = _load()
    x = _f32(x)
    weight = _f32(weight)
    b, d, L = x.shape
    W = weight.shape[1]
    assert weight.shape == (d, W)
    bb = None if bias is None else _f32(bias)
    out = np.empty((b, d, L), np.float64)
    lib.oracle_causal_conv1d(_ptr(x), _ptr(weight), _ptr(bb), _ptr(out),
                             b, d, L, W)
    return out


def gdn_chunk_fwd_h(k, w, u, g, h0=None, *, chunk_size: int = 64,
                    nthreads: int = 0) -> Dict[str, np.ndarray]:
    """Gated DeltaNet inter-chunk state pass in fp64.

    k, w [b, L, H, K]; u [b, L, H, V]; g [b, L, H] (chunk-local cumulative
    log-gates); h0 [b, H, K, V] or None.  Returns
      h      [b, H, NT, K, V]  state at the start of each chunk
      v_new  [b, L, H, V]      u - w h
      final  [b, H, K, V]
    """
    lib = _load()
    k, w, u, g = map(_f32, (k, w, u, g))
    b, L, H, K = k.shape
    V = u.shape[3]
    assert w.shape == k.shape and u.shape[:3] == (b, L, H) and g.shape == (b, L, H)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float64)
    nt = -(-L // chunk_size)
    h = np.empty((b, H, nt, K, V), np.float64)
    vn = np.empty((b, L, H, V), np.float64)
    fin = np.empty((b, H, K, V), np.float64)
    lib.oracle_gdn_chunk_fwd_h(_ptr(k), _ptr(w), _ptr(u), _ptr(g), _ptr(h0),
                               _ptr(h), _ptr(vn), _ptr(fin), b, L, H, K, V,
                               chunk_size, nthreads)
    return {"h": h, "v_new": vn, "final": fin}


def gdn_chunk_fwd_o(q, k, v_new, h, g, *, scale: float = 1.0,
                    chunk_size: int = 64, nthreads: int = 0) -> np.ndarray:
    """Gated DeltaNet output in fp64: q, k [b, L, H, K]; v_new [b, L, H, V]
    and h [b, H, NT, K, V] (any float type; used as doubles); g [b, L, H].
    Returns o [b, L, H, V]."""
    lib = _load()
    q, k, g = map(_f32, (q, k, g))
    v_new = np.ascontiguousarray(v_new, dtype=np.float64)
    h = np.ascontiguousarray(h, dtype=np.float64)
    b, L, H, K = q.shape
    V = v_new.shape[3]
    o = np.empty((b, L, H, V), np.float64)
    lib.oracle_gdn_chunk_fwd_o(_ptr(q), _ptr(k), _ptr(v_new), _ptr(h), _ptr(g),
                               _ptr(o), float(scale), b, L, H, K, V, chunk_size,
                               nthreads)
    return o
