"""The hot path inside a HIP graph.

ssd_forward (three kernel launches, no allocation, no memset) is captured
once in a HIP graph and replayed several times, with eager work and
synchronisations between the replays; every replay must reproduce the eager
call bit for bit.  The benchmark times the stage kernels from such replays.
"""
import numpy as np
import pytest
import torch

from gpu_util import device_inputs, log
from ssd_workloads import WORKLOADS, make_inputs, small_variant

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def ssd():
    import mamba_ssd_chunked_fwd_amd as m
    return m


# (workload, batch, seqlen, heads): the last is a long chain on few heads,
# for which the state pass runs as chunk_state + state_passing
GRAPH_CASES = [("small_bf16", 2, 300, None), ("wide_fp32", 2, 300, None),
               ("long_bf16", 1, 16384 + 77, 4)]


@pytest.mark.parametrize("name,batch,seqlen,heads", GRAPH_CASES,
                         ids=[c[0] + ("_two_level" if c[3] else "") for c in GRAPH_CASES])
def test_forward_replays_from_a_hip_graph(ssd, name, batch, seqlen, heads):
    w = small_variant(WORKLOADS[name], batch=batch, seqlen=seqlen,
                      **({"nheads": heads} if heads else {}))
    log(f"[graph] {w}")
    dev = device_inputs(make_inputs(w, seed=77), w.dtype)
    d = ssd.make_dims(dev["x"], dev["B"], w.chunk_size)
    b, L, H, P, N, nc = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.nchunks
    ws = torch.empty(ssd.workspace_bytes(d), dtype=torch.uint8, device=DEV)

    def outputs():
        return (torch.full((b, L, H, P), float("nan"), device=DEV),
                torch.full((b, H, nc, P, N), float("nan"), device=DEV),
                torch.full((b, H, P, N), float("nan"), device=DEV))

    def run(y, st, fin):
        ssd.ssd_forward(dev["x"], dev["dt"], dev["A"], dev["B"], dev["C"], dev["D"],
                        dev["init_state"], y, st, fin, ws, w.chunk_size)

    ref = outputs()
    run(*ref)
    torch.cuda.synchronize()
    got = outputs()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(*got)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in got:
            t.fill_(float("nan"))
        other = outputs()
        run(*other)                       # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        for a, r in zip(got, ref):
            assert torch.equal(a, r), rep
        for a, r in zip(other, ref):
            assert torch.equal(a, r), rep
