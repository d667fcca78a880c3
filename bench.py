"""Benchmark of the Mamba-2 SSD chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one ssd_forward call -- the whole hot path: stage 1 (chunk
cumsum), stage 2 (state pass), stage 3 (fused output) -- over one batch of
synthetic input of the named workload (default: the small-model bf16 layer,
batch 4 x 2048 tokens, 24 heads of 64, state 128, chunk 64).  The wall clock
over K steps gives tokens/s.  A second timed loop calls the three stage entry
points (ssd_chunk_cumsum, ssd_fwd_pass_state, ssd_compute_out) -- exactly the
kernels ssd_forward launches -- each captured in a HIP graph and replayed
between HIP events on the launch stream, which gives each kernel's mean
duration for the per-stage lines and the roofline.

Inputs are resident in HBM before timing.  Steps rotate over several
independent input/output sets whose total footprint is >= 1 GiB, so no step
finds its operands in the 256 MB last-level cache from the previous step.

Prints ONE JSON line: tokens/s (whole job), the roofline of the dominant
kernel from algorithmic bytes and its event-measured duration, and the fp64
CPU oracle timed on this host as a reported baseline.  Side fields (not part
of the step): the streaming decode step at the workload's batch and heads,
the causal conv1d that feeds the layer's SSD, and the Gated DeltaNet
chunk_fwd_h / chunk_fwd_o kernels on their own layer shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SSD forward tokens/sec + % of HBM/MFMA roofline, 1×MI355X"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_MFMA_TFLOPS = 2500.0      # dense
FP32_MFMA_TFLOPS = 157.3
# the kernel sources of each stage (the state pass runs as one kernel or as
# chunk_state + state_passing, chosen by shape)
STAGE_SOURCES = {"chunk_cumsum": ["ssd_chunk_cumsum.hip"],
                 "fwd_pass_state": ["ssd_fwd_pass_state.hip", "ssd_state_two_level.hip"],
                 "compute_out": ["ssd_compute_out.hip"]}


def algorithmic(w, y_bytes: int):
    """Bytes each stage must move and FLOPs it must do (no redundancy, no
    masked upper triangle), per launch over the whole workload."""
    b, L, H, P, N, G, T = (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                           w.ngroups, w.chunk_size)
    e = 2 if w.dtype == "bf16" else 4
    nc = w.nchunks
    init = 1 if w.init_std is not None else 0
    by = {
        "chunk_cumsum": 12 * b * L * H,
        "fwd_pass_state": (e * b * L * H * P + e * b * L * G * N + 8 * b * L * H
                           + 4 * b * H * P * N * init + 4 * b * H * nc * P * N
                           + 4 * b * H * P * N),
        "compute_out": (e * b * L * H * P + 2 * e * b * L * G * N + 8 * b * L * H
                        + 4 * b * H * nc * P * N + 4 * H + y_bytes * b * L * H * P),
    }
    fl = {
        "chunk_cumsum": 2 * b * L * H,
        "fwd_pass_state": 2 * b * L * H * P * N,
        "compute_out": (2 * b * L * H * P * N + b * nc * H * T * (T + 1) * P
                        + b * nc * G * T * (T + 1) * N),
    }
    return by, fl


def source_sha(stage: str) -> str:
    h = hashlib.sha256()
    for name in STAGE_SOURCES[stage]:
        with open(os.path.join(ROOT, "mamba_ssd_chunked_fwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(stage):
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_baseline(w, inp, min_seconds: float = 10.0):
    """The fp64 oracle on the host cores, over the full workload, repeated
    until about `min_seconds` of CPU work (at least 3 runs)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if threads <= 0:
        threads = len(os.sched_getaffinity(0))
    times = []
    while len(times) < 3 or (sum(times) < min_seconds and len(times) < 1000):
        t0 = time.perf_counter()
        oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                       inp["D"], inp["init_state"], chunk_size=w.chunk_size,
                       nthreads=threads)
        times.append(time.perf_counter() - t0)
    total = sum(times)
    return {"value": w.tokens * len(times) / total, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": (f"the full {w.name} workload ({w.batch * w.nheads} "
                       f"(batch, head) pairs x {w.seqlen} tokens), fp64 "
                       f"token recurrence, OpenMP over pairs; {len(times)} runs, "
                       f"{total:.1f} s in total (median run {statistics.median(times):.3f} s)")}


def gdn_bench(ssd, c, make, dev, stream, nrep):
    """Event-timed chunk_fwd_h and chunk_fwd_o over two rotating input sets
    (each larger than the 256 MB last-level cache)."""
    import torch
    inp = make(c, seed=3)
    b, L, H, K, V, nt = c.batch, c.seqlen, c.nheads, c.dk, c.dv, c.nchunks
    bf = torch.bfloat16

    def one_set():
        s = {k: torch.from_numpy(inp[k]).to(dev, bf) for k in ("q", "k", "w", "u")}
        s["g"] = torch.from_numpy(inp["g"]).to(dev)
        s["h"] = torch.empty(b, H, nt, K, V, device=dev)
        s["vn"] = torch.empty(b, L, H, V, device=dev, dtype=bf)
        s["fin"] = torch.empty(b, H, K, V, device=dev)
        s["o"] = torch.empty(b, L, H, V, device=dev, dtype=bf)
        return s
    sets = [one_set() for _ in range(2)]

    def fh(s):
        ssd.ssd_gdn_chunk_fwd_h(s["k"], s["w"], s["u"], s["g"], None, s["h"], s["vn"], s["fin"])

    def fo(s):
        ssd.ssd_gdn_chunk_fwd_o(s["q"], s["k"], s["vn"], s["h"], s["g"], s["o"], 1.0)
    for i in range(4):
        fh(sets[i % 2])
        fo(sets[i % 2])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nrep)]
    torch.cuda.synchronize()
    for i in range(nrep):
        ev[i][0].record(stream)
        fh(sets[i % 2])
        ev[i][1].record(stream)
        fo(sets[i % 2])
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    h_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in ev)
    o_ms = statistics.mean(e[1].elapsed_time(e[2]) for e in ev)
    e = 2
    h_bytes = (2 * e * b * L * H * K + e * b * L * H * V + 4 * b * L * H + 4 * b * H * nt * K * V
               + e * b * L * H * V + 4 * b * H * K * V)
    o_bytes = (2 * e * b * L * H * K + e * b * L * H * V + 4 * b * H * nt * K * V + 4 * b * L * H
               + e * b * L * H * V)

    def line(ms, by):
        gbs = by / (ms * 1e-3) / 1e9
        return {"ms": round(ms, 5), "alg_bytes": by, "GB_per_s": round(gbs, 1),
                "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    del sets
    return {"workload": {"name": c.name, "batch": b, "seqlen": L, "nheads": H, "dk": K,
                         "dv": V, "chunk_size": c.chunk_size, "dtype": c.dtype},
            "chunk_fwd_h": line(h_ms, h_bytes), "chunk_fwd_o": line(o_ms, o_bytes),
            "tokens_per_s": round(b * L / ((h_ms + o_ms) * 1e-3), 1),
            "note": "w, u synthetic (the WY transform is not on this path); bf16 v_new and o"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="small_bf16")
    ap.add_argument("--y-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gdn", action="store_true",
                    help="skip the Gated DeltaNet kernels' timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter scale)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              "is not supported (the path shards over (batch, head) with no "
              "communication between GPUs).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import mamba_ssd_chunked_fwd_amd as ssd
    from ssd_workloads import (GDN_WORKLOADS, WORKLOADS, conv_workload_for,
                               make_conv_inputs, make_gdn_inputs, make_inputs)

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(w)
    tin = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    ty = torch.bfloat16 if args.y_dtype == "bf16" else torch.float32
    b, L, H, P, N, G, T = (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                           w.ngroups, w.chunk_size)
    nc = w.nchunks
    y_bytes = 2 if ty == torch.bfloat16 else 4
    by, fl = algorithmic(w, y_bytes)
    set_bytes = by["fwd_pass_state"] + by["compute_out"]
    nsets = max(1, min(16, -(-(1 << 30) // set_bytes)))

    d = ssd.SsdDims(b, L, H, P, N, G, T)
    ws_bytes = ssd.workspace_bytes(d)

    def make_set():
        s = {k: torch.from_numpy(inp[k]).to(dev, tin) for k in ("x", "B", "C")}
        for k in ("dt", "A", "D"):
            s[k] = torch.from_numpy(inp[k]).to(dev)
        s["init"] = (None if inp["init_state"] is None
                     else torch.from_numpy(inp["init_state"]).to(dev))
        s["ws"] = torch.empty(-(-ws_bytes // 4), device=dev)  # ssd_forward's workspace
        s["g"] = s["ws"][: b * H * L].view(b, H, L)
        s["dt_t"] = s["ws"][b * H * L: 2 * b * H * L].view(b, H, L)
        s["states"] = torch.empty(b, H, nc, P, N, device=dev)
        s["final"] = torch.empty(b, H, P, N, device=dev)
        s["y"] = torch.empty(b, L, H, P, device=dev, dtype=ty)
        return s

    sets = [make_set() for _ in range(nsets)]
    stream = torch.cuda.current_stream(dev)

    def forward(s):
        ssd.ssd_forward(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"],
                        s["init"], s["y"], s["states"], s["final"], s["ws"], T)

    # ---- the step: ssd_forward, the whole hot path, as a user calls it
    for i in range(args.warmup):
        forward(sets[i % nsets])
    # the timed steps carry no events between them: nothing but the step's
    # own launches reaches the stream inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        forward(sets[i % nsets])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the same step bracketed by HIP events, in a loop of its own
    nfe = max(20, args.steps // 2)
    fwd_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(nfe)]
    torch.cuda.synchronize()
    for i in range(nfe):
        fwd_ev[i][0].record(stream)
        forward(sets[i % nsets])
        fwd_ev[i][1].record(stream)
    torch.cuda.synchronize()
    fwd_ms = statistics.mean(e[0].elapsed_time(e[1]) for e in fwd_ev)

    # ---- every entry point on its own, HIP events on the launch stream
    def stage_calls(s):
        return [
            ("chunk_cumsum", lambda: ssd.ssd_chunk_cumsum(s["dt"], s["A"], s["g"],
                                                          s["dt_t"], T)),
            ("fwd_pass_state", lambda: ssd.ssd_fwd_pass_state(
                s["x"], s["B"], s["dt_t"], s["g"], s["init"], s["states"],
                s["final"], T)),
            ("compute_out", lambda: ssd.ssd_compute_out(
                s["x"], s["B"], s["C"], s["dt_t"], s["g"], s["states"], s["D"],
                s["y"], T)),
        ]
    stage_names = [n for n, _ in stage_calls(sets[0])]
    nst = max(20, args.steps // 2)
    for i in range(5):
        for _, f in stage_calls(sets[i % nsets]):
            f()
    # Each entry point's nst launches (over the rotating sets, whose inputs
    # the warm-up steps produced) are captured once in a HIP graph; the graph
    # is replayed between two HIP events, so the mean launch duration holds
    # neither host launch time nor an event between launches.  (Eager loops
    # with one event per launch add about 3 us per launch; the short first
    # stage is then host-bound.)
    dur = {}
    for k, n in enumerate(stage_names):
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            for i in range(nst):
                stage_calls(sets[i % nsets])[k][1]()
        sg.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(3):
            sg.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        dur[n] = e0.elapsed_time(e1) / (3 * nst)
        del sg

    # ---- the streaming decode step at the same batch and heads: one token
    #      per sequence from the carried state (read and written in place)
    dec_states = [torch.randn(b, H, P, N, device=dev) for _ in range(nsets)]
    dec_in = [(s["x"][:, 0].contiguous(), s["dt"][:, 0].contiguous(),
               s["B"][:, 0].contiguous(), s["C"][:, 0].contiguous(),
               torch.empty(b, H, P, device=dev, dtype=ty)) for s in sets]
    for i in range(5):
        xt, dtt, Bt, Ct, yt = dec_in[i % nsets]
        ssd.ssd_decode_step(xt, dtt, sets[0]["A"], Bt, Ct, sets[0]["D"],
                            dec_states[i % nsets], yt)
    # A decode step is a few microseconds of GPU work, less than the host
    # needs to issue one through Python, so an eager loop would time the
    # host.  The steps are captured once in a HIP graph and the graph is
    # replayed between two events (each replay = ndec steps back to back).
    ndec, nrep_dec = 50, 8
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        for i in range(ndec):
            xt, dtt, Bt, Ct, yt = dec_in[i % nsets]
            ssd.ssd_decode_step(xt, dtt, sets[0]["A"], Bt, Ct, sets[0]["D"],
                                dec_states[i % nsets], yt)
    dgraph.replay()
    dec_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    dec_ev[0].record(stream)
    for _ in range(nrep_dec):
        dgraph.replay()
    dec_ev[1].record(stream)
    torch.cuda.synchronize()
    dec_ms = dec_ev[0].elapsed_time(dec_ev[1]) / (nrep_dec * ndec)
    del dgraph
    dec_bytes = (8 * b * H * P * N + (2 if w.dtype == "bf16" else 4) * (b * H * P + 2 * b * G * N)
                 + 4 * b * H + 8 * H + y_bytes * b * H * P)

    # ---- the causal depthwise conv1d that feeds this layer's SSD (over the
    #      x, B and C channels), x and out in the workload's storage type
    cw = conv_workload_for(w)
    cinp = make_conv_inputs(cw, seed=7)
    cx0 = torch.from_numpy(cinp["x"]).to(dev, tin)
    cwt = torch.from_numpy(cinp["weight"]).to(dev)
    cbias = torch.from_numpy(cinp["bias"]).to(dev)
    cset_bytes = 2 * cx0.numel() * cx0.element_size()
    nconv = max(2, min(16, -(-(1 << 30) // cset_bytes)))
    conv_sets = [((cx0 if i == 0 else cx0.clone()), torch.empty_like(cx0)) for i in range(nconv)]
    for i in range(5):
        cx, co = conv_sets[i % nconv]
        ssd.ssd_causal_conv1d(cx, cwt, cbias, co)
    nconv_steps = max(50, args.steps)
    conv_ev = [torch.cuda.Event(enable_timing=True) for _ in range(nconv_steps + 1)]
    torch.cuda.synchronize()
    conv_ev[0].record(stream)
    for i in range(nconv_steps):
        cx, co = conv_sets[i % nconv]
        ssd.ssd_causal_conv1d(cx, cwt, cbias, co)
        conv_ev[i + 1].record(stream)
    torch.cuda.synchronize()
    conv_ms = statistics.mean(conv_ev[i].elapsed_time(conv_ev[i + 1])
                              for i in range(nconv_steps))
    conv_bytes = cset_bytes + 4 * cw.dim * (cw.width + 1)
    del conv_sets

    # ---- Gated DeltaNet chunked forward (chunk_fwd_h then chunk_fwd_o) on
    #      its own layer shape, v_new and o in bf16
    gdn = gdn_bench(ssd, GDN_WORKLOADS["gdn_layer_bf16"], make_gdn_inputs, dev, stream,
                    max(20, args.steps // 2)) if not args.no_gdn else None

    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()

    # The practical streaming ceiling of this GPU in the same run: a 1 GiB
    # device-to-device copy (read + write), timed from a graph of 5 copies.
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        for _ in range(5):
            cdst.copy_(csrc)
    cg.replay()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ce[0].record(stream)
    cg.replay()
    ce[1].record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 5 / (ce[0].elapsed_time(ce[1]) * 1e-3) / 1e9
    del cg, csrc, cdst

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = w.tokens / (wall / args.steps)
    peak_tf = BF16_MFMA_TFLOPS if w.dtype == "bf16" else FP32_MFMA_TFLOPS
    stages = {}
    for n in stage_names:
        ms = dur[n]
        gbs = by[n] / (ms * 1e-3) / 1e9
        stages[n] = {"ms": round(ms, 5), "alg_bytes": by[n], "alg_flop": fl[n],
                     "GB_per_s": round(gbs, 1),
                     "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
                     "frac_of_copy": round(gbs / copy_gbs, 4),
                     "TFLOP_per_s": round(fl[n] / (ms * 1e-3) / 1e12, 2),
                     "mfma_frac_of_peak": round(fl[n] / (ms * 1e-3) / 1e12 / peak_tf, 4)}
    # the kernels one ssd_forward call launches
    step_kernels = ["chunk_cumsum", "fwd_pass_state", "compute_out"]
    dom = max(step_kernels, key=lambda n: dur[n])
    achieved = by[dom] / (dur[dom] * 1e-3) / 1e9
    traffic = measured_traffic(w.name, dom)
    step_bytes = sum(by[n] for n in step_kernels)
    total_flop = sum(fl[n] for n in step_kernels)
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "batch": b, "seqlen": L, "nheads": H,
                   "headdim": P, "dstate": N, "ngroups": G, "chunk_size": T,
                   "x_dtype": w.dtype, "y_dtype": args.y_dtype,
                   "state_dtype": "fp32", "input_sets_rotated": nsets},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "stages": stages,
        "ssd_forward_event_ms": round(fwd_ms, 5),
        "decode_step": {"ms": round(dec_ms, 5), "tokens_per_s": round(b / (dec_ms * 1e-3), 1),
                        "alg_bytes": dec_bytes,
                        "GB_per_s": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "note": "one token for each of the batch's sequences, state in place; "
                                "steps replayed from a HIP graph; the rotated states "
                                f"({nsets} x {4 * b * H * P * N / 1e6:.1f} MB) stay in the "
                                "last-level cache"},
        "causal_conv1d": {"ms": round(conv_ms, 5),
                          "shape": {"batch": cw.batch, "dim": cw.dim, "seqlen": cw.seqlen,
                                    "width": cw.width, "dtype": cw.dtype},
                          "alg_bytes": conv_bytes,
                          "GB_per_s": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "the conv over the layer's x, B, C channels; not part of the step"},
        "gated_deltanet": gdn,
        "copy_GB_per_s": round(copy_gbs, 1),
        "effective_TFLOP_per_s": round(total_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "hbm_floor_ms": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e3, 5),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
