"""Seeded synthetic inputs for the Mamba-2 SSD chunked forward.

This module only draws random numbers and rounds them to the storage type.
It holds none of the method's arithmetic (no decay, cumsum, state or output
math), so the CPU oracle and the HIP path can both be fed from it without
sharing any of the computation under test.

Workloads
---------
The five named workloads below fix shapes and value distributions.  The
distributions follow the domain the pages state for the recurrence's inputs
("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
CUDA Tile", section "The Mamba-2 Recurrence": dt is positive, A is negative,
so exp(A*dt) lies in (0, 1]).  dt arrives already passed through softplus; the
method applies no further preprocessing to it.

Draw order (fixed, one ``numpy.random.Generator(PCG64(seed))`` per workload):
x, B, C, z_dt, u_A, D, init_state.  bf16 tensors are float32 draws rounded to
bfloat16 with round-to-nearest-even, then held as float32 (every bf16 value
is exactly representable in float32), so both sides read identical values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional, Tuple

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int      # P: size of x_t per head
    dstate: int       # N: size of B_t and C_t (the state size)
    ngroups: int      # G: B and C are shared by nheads/ngroups heads
    chunk_size: int   # T
    dtype: str        # "fp32" or "bf16": storage type of x, B, C
    dt_shift: float   # dt = softplus(N(0,1) + dt_shift)
    a_low: float      # A = -exp(U(a_low, a_high))
    a_high: float
    init_std: Optional[float]  # None: zero initial state

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    # Tiny fp32 case the oracle finishes instantly.
    "tiny_fp32": Workload("tiny_fp32", 1, 256, 2, 64, 64, 1, 64, "fp32",
                          -2.0, 0.0, 1.5, None),
    # Small-model layer (d_model 768, expand 2 -> 24 heads of 64).
    "small_bf16": Workload("small_bf16", 4, 2048, 24, 64, 128, 1, 64, "bf16",
                           -2.0, 0.0, 1.5, None),
    # Large-model layer (d_model 2560, expand 2 -> 80 heads of 64).
    "large_bf16": Workload("large_bf16", 2, 8192, 80, 64, 128, 1, 256, "bf16",
                           -2.0, 0.0, 1.5, None),
    # Long-sequence streaming prefill with a carried-in state.
    "long_bf16": Workload("long_bf16", 1, 65536, 32, 64, 128, 1, 128, "bf16",
                          -2.0, 0.0, 1.5, 0.1),
    # Wide batch, grouped B/C (8 groups of 6 heads), stronger decay, fp32.
    "wide_fp32": Workload("wide_fp32", 64, 1024, 48, 64, 64, 8, 64, "fp32",
                          -1.0, -1.0, 2.0, None),
}

# Seeds are fixed per workload so every consumer draws the same arrays.
SEEDS: Dict[str, int] = {"tiny_fp32": 1, "small_bf16": 2, "large_bf16": 3,
                         "long_bf16": 4, "wide_fp32": 5}


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return float32.

    Finite inputs only (the generators never produce NaN or Inf).
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _softplus(z: np.ndarray) -> np.ndarray:
    # log(1 + e^z), computed without overflow.
    return np.logaddexp(0.0, z)


def make_inputs(w: Workload, seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw the inputs of workload ``w``.

    Returns float32 numpy arrays, contiguous, in the layouts the method uses:
      x     [batch, seqlen, nheads, headdim]
      B, C  [batch, seqlen, ngroups, dstate]
      dt    [batch, seqlen, nheads]
      A, D  [nheads]
      init_state [batch, nheads, headdim, dstate] or None
    For bf16 workloads x, B, C hold bf16-representable values.
    """
    if seed is None:
        seed = SEEDS.get(w.name, 0)
    rng = np.random.Generator(np.random.PCG64(seed))
    b, L, H, P, N, G = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups
    x = rng.standard_normal((b, L, H, P), dtype=np.float32)
    B = rng.standard_normal((b, L, G, N), dtype=np.float32)
    C = rng.standard_normal((b, L, G, N), dtype=np.float32)
    z = rng.standard_normal((b, L, H), dtype=np.float32)
    u = rng.uniform(w.a_low, w.a_high, size=H)
    D = rng.standard_normal(H).astype(np.float32)
    init = None
    if w.init_std is not None:
        init = (rng.standard_normal((b, H, P, N), dtype=np.float32)
                * np.float32(w.init_std))
    dt = _softplus(z.astype(np.float64) + w.dt_shift).astype(np.float32)
    A = (-np.exp(u)).astype(np.float32)
    if w.dtype == "bf16":
        x, B, C = round_to_bf16(x), round_to_bf16(B), round_to_bf16(C)
    elif w.dtype != "fp32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    return {"x": x, "B": B, "C": C, "dt": dt, "A": A, "D": D,
            "init_state": init}


@dataclasses.dataclass(frozen=True)
class ConvWorkload:
    """Shape of the Mamba block's causal depthwise conv1d, x [batch, dim,
    seqlen].  In a Mamba-2 layer the conv runs over the channels that become
    x, B and C: dim = nheads * headdim + 2 * ngroups * dstate."""
    name: str
    batch: int
    dim: int
    seqlen: int
    width: int
    dtype: str        # storage type of x (and of the output the bench times)
    bias: bool = True


def conv_workload_for(w: Workload, width: int = 4) -> ConvWorkload:
    """The conv1d that feeds workload ``w``'s SSD (same batch, seqlen, dtype)."""
    dim = w.nheads * w.headdim + 2 * w.ngroups * w.dstate
    return ConvWorkload("conv_" + w.name, w.batch, dim, w.seqlen, width, w.dtype)


def make_conv_inputs(c: ConvWorkload, seed: int = 0) -> Dict[str, np.ndarray]:
    """Draw x [batch, dim, seqlen] ~ N(0, 1) (rounded to bf16 for bf16
    workloads), weight [dim, width] and bias [dim] ~ U(-k, k), k =
    1/sqrt(width) (the fan-in scale of a depthwise filter).  Draw order: x,
    weight, bias.  Returns float32 arrays; bias is None without a bias."""
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal((c.batch, c.dim, c.seqlen), dtype=np.float32)
    k = 1.0 / np.sqrt(c.width)
    weight = rng.uniform(-k, k, size=(c.dim, c.width)).astype(np.float32)
    bias = rng.uniform(-k, k, size=c.dim).astype(np.float32)
    if c.dtype == "bf16":
        x = round_to_bf16(x)
    elif c.dtype != "fp32":
        raise ValueError(f"unknown dtype {c.dtype!r}")
    return {"x": x, "weight": weight, "bias": bias if c.bias else None}


@dataclasses.dataclass(frozen=True)
class GdnWorkload:
    """Shape of a Gated DeltaNet layer's chunked forward: q, k, w
    [batch, seqlen, nheads, dk]; u [batch, seqlen, nheads, dv]; chunks of 64."""
    name: str
    batch: int
    seqlen: int
    nheads: int
    dk: int
    dv: int
    dtype: str = "bf16"
    init_std: Optional[float] = None
    chunk_size: int = 64

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen


GDN_WORKLOADS: Dict[str, GdnWorkload] = {
    # A 16-head GDN layer with 128-wide keys and values, 8 x 2048 tokens.
    "gdn_layer_bf16": GdnWorkload("gdn_layer_bf16", 8, 2048, 16, 128, 128),
}


def make_gdn_inputs(c: GdnWorkload, seed: int = 0) -> Dict[str, np.ndarray]:
    """Draw the chunked Gated DeltaNet inputs.

    Draw order: q, k, k2, v, beta, a, h0.  q ~ N(0, 1); k and k2 are N(0, 1)
    rows scaled to unit L2 norm; beta ~ U(0.1, 0.9); the per-token log-gates
    a ~ U(-0.5, -0.01).  The kernels take the WY-transformed keys and values
    as inputs, so w and u are drawn with the same shapes and scale: w_t =
    beta_t k2_t (a unit row independent of k_t) and u_t = beta_t v_t.  g, the
    gate input, is the chunk-local running sum of a (float64, then float32),
    the form the chunked kernels read.  q, k, w, u are rounded to bf16 for
    bf16 workloads.  h0 ~ N(0, init_std) or None.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    b, L, H, K, V, C = c.batch, c.seqlen, c.nheads, c.dk, c.dv, c.chunk_size
    q = rng.standard_normal((b, L, H, K), dtype=np.float32)
    k = rng.standard_normal((b, L, H, K), dtype=np.float32)
    k2 = rng.standard_normal((b, L, H, K), dtype=np.float32)
    v = rng.standard_normal((b, L, H, V), dtype=np.float32)
    beta = rng.uniform(0.1, 0.9, size=(b, L, H)).astype(np.float32)
    a = rng.uniform(-0.5, -0.01, size=(b, L, H))
    h0 = None
    if c.init_std is not None:
        h0 = (rng.standard_normal((b, H, K, V), dtype=np.float32)
              * np.float32(c.init_std))
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    k2 = k2 / np.linalg.norm(k2, axis=-1, keepdims=True)
    w = beta[..., None] * k2
    u = beta[..., None] * v
    g = np.empty((b, L, H), np.float64)
    for t0 in range(0, L, C):
        g[:, t0:t0 + C] = np.cumsum(a[:, t0:t0 + C], axis=1)
    g = g.astype(np.float32)
    if c.dtype == "bf16":
        q, k, w, u = (round_to_bf16(x) for x in (q, k, w, u))
    elif c.dtype != "fp32":
        raise ValueError(f"unknown dtype {c.dtype!r}")
    f = lambda x: np.ascontiguousarray(x, dtype=np.float32)
    return {"q": f(q), "k": f(k), "w": f(w), "u": f(u), "g": f(g), "h0": h0}


def small_variant(w: Workload, **kw) -> Workload:
    """A reduced copy of ``w`` (same dtype and distributions)."""
    return w.with_(name=w.name + "_small", **kw)


def shape_tuple(w: Workload) -> Tuple[int, ...]:
    return (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups,
            w.chunk_size)
