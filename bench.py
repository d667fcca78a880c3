"""Benchmark of the Mamba-2 SSD chunked forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-configs] [--no-cpu-baseline] [--no-side]

A step is one ssd_forward call -- the whole hot path: stage 1 (chunk
cumsum), stage 2 (state pass), stage 3 (fused output) -- over one batch of
synthetic input of the named workload.  For fp32 inputs with 64-token chunks,
N = 64 and at least one (batch, head pair) per CU, ssd_forward runs stages 2
and 3 as one kernel (ssd_state_and_out); the step's kernels are then stage 1
and that one, and the two-kernel path is timed beside it for reference.  The default workload is the largest
of the five (wide_fp32: 64 sequences of 1024 tokens, 48 heads, 8 groups,
state 64, fp32; 4.6 GB of algorithmic traffic per step).  The wall clock
over K steps gives `value` in tokens/s.

Per-kernel durations come from HIP graphs: each stage entry point's launches
(over the rotating input sets) are captured once and the graph is replayed
between two HIP events on the launch stream, so a duration holds neither
host launch time nor an event between launches.  They give the per-stage
lines and the roofline of the dominant kernel: algorithmic bytes per launch
(the method's inputs and outputs, each moved once) over the mean duration,
against the MI355X HBM peak of 8 TB/s.

The `configs` map repeats the graph timing (ssd_forward and each stage) for
all five workloads, so every configuration has a number from this run.

Inputs are resident in HBM before timing.  Steps rotate over independent
input/output sets whose total footprint is >= 1 GiB, so no step finds its
operands in the 256 MB last-level cache from the previous step.

Prints ONE JSON line.  Side fields (not part of the step): the streaming
decode step at the workload's batch and heads, the causal conv1d that feeds
the layer's SSD, and the Gated DeltaNet chunk_fwd_h / chunk_fwd_o kernels on
their own layer shape.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
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
CONFIG_ORDER = ["tiny_fp32", "small_bf16", "large_bf16", "long_bf16", "wide_fp32"]
# the kernel sources of each stage (the state pass runs as one kernel or as
# chunk_state + state_passing, chosen by shape)
STAGE_SOURCES = {"chunk_cumsum": ["ssd_chunk_cumsum.hip"],
                 "fwd_pass_state": ["ssd_fwd_pass_state.hip", "ssd_state_two_level.hip",
                                    "ssd_state_pair_f32.hip"],
                 "compute_out": ["ssd_compute_out.hip"],
                 "state_and_out": ["ssd_fused_f32.hip", "ssd_fused_bf16.hip"]}
THREE_STAGES = ["chunk_cumsum", "fwd_pass_state", "compute_out"]
FUSED_STAGES = ["chunk_cumsum", "state_and_out"]


def heads_per_pair(w) -> int:
    return 2 if (w.nheads // w.ngroups) % 2 == 0 else 1


def fused(w, cus: int = 256) -> bool:
    """Whether ssd_forward runs stages 2 and 3 as one pass for this
    workload (the library's own rule): fp32 with 64-token chunks, N = 64 and
    a (batch, head pair) per CU; or bf16 with N = 128 and an even group
    size."""
    if w.dtype == "fp32":
        return (w.chunk_size == 64 and w.dstate == 64
                and w.batch * w.nheads // heads_per_pair(w) >= cus)
    return (w.dstate == 128 and w.headdim == 64 and w.chunk_size in (64, 128, 256)
            and (w.nheads // w.ngroups) % 2 == 0)


def run_plan(w, cus: int = 256) -> dict:
    """The bf16 fused pass's cut of each chain into runs (the library's own
    rule): R = the chunk steps per CU if the walk were spread evenly, a lead
    run of R0 = nc - (nr - 1) R chunks and nr - 1 runs of R; the run pass
    walks every run but the last."""
    nc = w.nchunks
    pairs = w.batch * w.nheads // 2
    per = -(-pairs * nc // cus)
    if per >= nc:
        nr, R, R0 = 1, nc, nc
    else:
        R = per
        nr = 1 + (nc - 1) // R
        R0 = nc - (nr - 1) * R
    return {"runs": nr, "run_chunks": R, "lead_chunks": R0,
            "run_pass_chunks": nc - R if nr > 1 else 0}


def step_kernels(w, cus: int = 256) -> list:
    return FUSED_STAGES if fused(w, cus) else THREE_STAGES


def algorithmic(w, y_bytes: int):
    """Bytes each stage must move and FLOPs it must do (no redundancy, no
    masked upper triangle), per launch over the whole workload.

    Stage 1 counts dt in and g out (8 bytes per (token, head)); the
    head-major copy of dt it also writes is a design choice of this
    implementation and is reported apart (`design_extra_bytes`)."""
    b, L, H, P, N, G, T = (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                           w.ngroups, w.chunk_size)
    e = 2 if w.dtype == "bf16" else 4
    nc = w.nchunks
    init = 1 if w.init_std is not None else 0
    by = {
        "chunk_cumsum": 8 * b * L * H,
        "fwd_pass_state": (e * b * L * H * P + e * b * L * G * N + 8 * b * L * H
                           + 4 * b * H * P * N * init + 4 * b * H * nc * P * N
                           + 4 * b * H * P * N),
        "compute_out": (e * b * L * H * P + 2 * e * b * L * G * N + 8 * b * L * H
                        + 4 * b * H * nc * P * N + 4 * H + y_bytes * b * L * H * P),
        # stages 2 and 3 in one pass: x, B, C, dt_t and g read once, the
        # states written and never read back
        "state_and_out": (e * b * L * H * P + 2 * e * b * L * G * N + 8 * b * L * H
                          + 4 * b * H * P * N * init + 4 * b * H * nc * P * N
                          + 4 * b * H * P * N + 4 * H + y_bytes * b * L * H * P),
    }
    fl = {
        "chunk_cumsum": 2 * b * L * H,
        "fwd_pass_state": 2 * b * L * H * P * N,
        "compute_out": (2 * b * L * H * P * N + b * nc * H * T * (T + 1) * P
                        + b * nc * G * T * (T + 1) * N),
    }
    fl["state_and_out"] = fl["fwd_pass_state"] + fl["compute_out"]
    return by, fl


def design_extra_bytes(w) -> dict:
    """Bytes a stage moves beyond the algorithmic count by design: stage 1's
    head-major copy of dt (read back by stages 2 and 3 in place of dt)."""
    return {"chunk_cumsum": 4 * w.batch * w.seqlen * w.nheads}


def state_pair(w, cus: int = 256) -> bool:
    """Whether stage 2 runs the fp32 head-pair kernel (the library's own
    rule): fp32 inputs, 64-token chunks, N = 64, an even group size and a
    (batch, head pair) per CU."""
    return (w.dtype == "fp32" and w.chunk_size == 64 and w.dstate == 64
            and (w.nheads // w.ngroups) % 2 == 0 and w.batch * w.nheads // 2 >= cus)


def mfma_kind(w) -> dict:
    """The matrix instruction each stage issues: bf16 (16x16x32) or fp32
    (16x16x4).  fp32 inputs run stage 3 on bf16 instructions (three-term
    splits) for chunks of up to 128 tokens, and stage 2 where the head-pair
    kernel applies."""
    out_bf16 = w.dtype == "bf16" or w.chunk_size <= 128
    return {"fwd_pass_state": "bf16" if w.dtype == "bf16" or state_pair(w) else "fp32",
            "compute_out": "bf16" if out_bf16 else "fp32",
            "state_and_out": "bf16"}


def issued_mfma_flop(w) -> dict:
    """Matrix-instruction work the kernels issue, from their structure:
    causal blocks on or below the diagonal in 16-row (and, on bf16
    instructions, 32-token) steps; with bf16 inputs, two instructions (hi +
    lo) for every product with a computed fp32 operand; with fp32 inputs on
    bf16 instructions, six per product (three-term splits of both
    operands).  C B^T is counted once per (batch, chunk, group)."""
    b, L, H, P, N, G, T = (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate,
                           w.ngroups, w.chunk_size)
    nc = w.nchunks
    nib = T // 16
    lx32 = sum(ib // 2 + 1 for ib in range(nib)) * 32 * 16 * P * 2   # 32-token k-steps
    lx16 = sum(ib + 1 for ib in range(nib)) * 16 * 16 * P * 2        # 16-token blocks
    cb = sum(ib + 1 for ib in range(nib)) * 16 * 16 * N * 2
    if w.dtype == "bf16":
        out = b * nc * H * (2 * 2 * T * P * N + 2 * lx32) + b * nc * G * cb
        a2 = 2 * (2 * b * L * H * P * N)                          # P^T: w o x hi + lo
    elif mfma_kind(w)["compute_out"] == "bf16":
        out = 6 * (b * nc * H * (2 * T * P * N + lx32) + b * nc * G * cb)
        # the head-pair state kernel: six bf16 products per fp32 product,
        # over whole 64-token chunks
        a2 = (6 * 2 * b * nc * T * H * P * N if state_pair(w)
              else 2 * b * L * H * P * N)
    else:
        out = b * nc * H * (2 * T * P * N + lx16) + b * nc * G * cb
        a2 = 2 * b * L * H * P * N
    if w.dtype == "fp32":
        # the fused pass (fp32 on bf16 instructions, six per product): C S^T,
        # X^T L'^T and the state update per (batch, chunk, head), C B^T once
        # per (batch, chunk, work item of heads_per_pair heads)
        fused_issued = 6 * (b * nc * H * (2 * 2 * T * P * N + lx32)
                            + b * nc * (H // heads_per_pair(w)) * cb)
    else:
        # the bf16 fused pass, per 64-token block of each (batch, head): C S^T
        # and the update with hi + lo of S and of w o x, X^T L'^T with hi + lo
        # of L' (six 32-token k-steps), C B^T once per head pair (ten 16x16
        # blocks); plus the run pass over the runs before the last (update only)
        nblk = -(-L // 64)
        lx64 = sum(ib // 2 + 1 for ib in range(4)) * 32 * 16 * P * 2
        cb64 = 10 * 16 * 16 * N * 2
        per_block = 2 * (2 * 64 * P * N) * 2 + 2 * lx64
        pl = run_plan(w)
        run_pass = b * H * pl["run_pass_chunks"] * (T // 64) * 2 * (2 * 64 * P * N)
        fused_issued = b * H * nblk * per_block + b * (H // 2) * nblk * cb64 + run_pass
    return {"fwd_pass_state": a2, "compute_out": out, "state_and_out": fused_issued}


def source_sha(stage: str) -> str:
    h = hashlib.sha256()
    for name in STAGE_SOURCES[stage]:
        with open(os.path.join(ROOT, "mamba_ssd_chunked_fwd_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_profile(workload: str, stage: str, kind: str):
    """A committed counter summary (profiles/<stage>_<workload>_<kind>.json)
    if it was taken from the current kernel source, else None."""
    path = os.path.join(ROOT, "profiles", f"{stage}_{workload}_{kind}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(stage):
        return None
    return rec


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def cpu_baseline(w, inp, min_seconds: float = 10.0):
    """The fp64 oracle (the parity checker, untuned) on the host cores, over
    the full workload, repeated until about `min_seconds` of CPU work (at
    least 2 runs)."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    if threads <= 0:
        threads = len(os.sched_getaffinity(0))
    used = min(threads, w.batch * w.nheads)      # OpenMP over (batch, head) pairs
    times = []
    while len(times) < 2 or (sum(times) < min_seconds and len(times) < 1000):
        t0 = time.perf_counter()
        oracle.forward(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                       inp["D"], inp["init_state"], chunk_size=w.chunk_size,
                       nthreads=threads)
        times.append(time.perf_counter() - t0)
    total = sum(times)
    return {"value": round(w.tokens * len(times) / total, 1), "unit": "tokens/s",
            "cores": used, "kind": "oracle", "cpu_model": cpu_model(),
            "threads_requested": threads, "host_cpus": os.cpu_count(),
            "sample": (f"the full {w.name} workload ({w.batch * w.nheads} "
                       f"(batch, head) pairs x {w.seqlen} tokens), fp64 "
                       f"token recurrence, OpenMP over pairs; {len(times)} runs, "
                       f"{total:.1f} s in total (median run {statistics.median(times):.3f} s)")}


def graph_time_ms(calls, nrep: int = 3, settle_ms: float = 30.0) -> float:
    """Mean duration of one call: the calls are captured once in a HIP graph,
    the graph is replayed untimed until `settle_ms` have passed (at least
    once; the capture leaves the GPU idle, and its clocks take some
    milliseconds of work to come back to their steady state), then `nrep`
    times between two HIP events on the current stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in calls:
            f()
    t0 = time.perf_counter()
    while True:
        g.replay()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= settle_ms:
            break
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(nrep):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / (nrep * len(calls))
    del g
    return ms


class WorkloadRun:
    """Device input/output sets of one workload and the calls that use them."""

    def __init__(self, ssd, w, y_dtype, dev):
        import torch
        from ssd_workloads import make_inputs
        self.ssd, self.w, self.dev = ssd, w, dev
        self.inp = make_inputs(w)
        inp = self.inp
        tin = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        self.y_bytes = 2 if y_dtype == torch.bfloat16 else 4
        self.by, self.fl = algorithmic(w, self.y_bytes)
        b, L, H, P, N, T = w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.chunk_size
        nc = w.nchunks
        self.kernels = step_kernels(w, torch.cuda.get_device_properties(dev).multi_processor_count)
        set_bytes = self.by["fwd_pass_state"] + self.by["compute_out"]
        self.nsets = max(1, min(16, -(-(1 << 30) // set_bytes)))
        d = ssd.SsdDims(b, L, H, P, N, w.ngroups, T)
        ws_bytes = ssd.workspace_bytes(d)
        base = {k: torch.from_numpy(inp[k]).to(dev, tin) for k in ("x", "B", "C")}
        for k in ("dt", "A", "D"):
            base[k] = torch.from_numpy(inp[k]).to(dev)
        base["init"] = (None if inp["init_state"] is None
                        else torch.from_numpy(inp["init_state"]).to(dev))

        def make_set(i):
            s = dict(base) if i == 0 else {k: (None if v is None else v.clone())
                                            for k, v in base.items()}
            s["ws"] = torch.empty(-(-ws_bytes // 4), device=dev)   # ssd_forward's workspace
            s["g"] = s["ws"][: b * H * L].view(b, H, L)
            s["dt_t"] = s["ws"][b * H * L: 2 * b * H * L].view(b, H, L)
            s["states"] = torch.empty(b, H, nc, P, N, device=dev)
            s["final"] = torch.empty(b, H, P, N, device=dev)
            s["y"] = torch.empty(b, L, H, P, device=dev, dtype=y_dtype)
            return s
        self.sets = [make_set(i) for i in range(self.nsets)]

    def forward(self, i):
        s = self.sets[i % self.nsets]
        self.ssd.ssd_forward(s["x"], s["dt"], s["A"], s["B"], s["C"], s["D"], s["init"],
                             s["y"], s["states"], s["final"], s["ws"], self.w.chunk_size)

    def stage(self, name, i):
        s, T, ssd = self.sets[i % self.nsets], self.w.chunk_size, self.ssd
        if name == "chunk_cumsum":
            ssd.ssd_chunk_cumsum(s["dt"], s["A"], s["g"], s["dt_t"], T)
        elif name == "fwd_pass_state":
            ssd.ssd_fwd_pass_state(s["x"], s["B"], s["dt_t"], s["g"], s["init"], s["states"],
                                   s["final"], T)
        elif name == "state_and_out":
            ssd.ssd_state_and_out(s["x"], s["B"], s["C"], s["dt_t"], s["g"], s["D"], s["init"],
                                  s["y"], s["states"], s["final"], T)
        else:
            ssd.ssd_compute_out(s["x"], s["B"], s["C"], s["dt_t"], s["g"], s["states"],
                                s["D"], s["y"], T)

    def time_all(self, nlaunch: int) -> dict:
        """Graph-replay durations (ms) of ssd_forward, of each of its
        kernels and, where stages 2 and 3 run fused, of the two-kernel path."""
        for i in range(max(3, self.nsets)):
            self.forward(i)
        out = {"ssd_forward": graph_time_ms([lambda i=i: self.forward(i)
                                             for i in range(nlaunch)])}
        names = list(dict.fromkeys(self.kernels + THREE_STAGES))
        for n in names:
            if n == "chunk_cumsum":
                continue
            out[n] = graph_time_ms([lambda i=i, n=n: self.stage(n, i) for i in range(nlaunch)])
        out.update(self.time_cumsum(nlaunch))
        return out

    def time_cumsum(self, nlaunch: int) -> dict:
        """Stage 1 over its own rotating dt / g / dt_t sets (>= 1 GiB in
        total, so no launch finds its operands in the last-level cache: the
        stage's footprint is a few tens of MB, which one set of the step's
        buffers would leave cache-resident), and two device-to-device copies
        over rotating buffers as its floor: one moving the stage's own bytes
        (dt read, g and dt_t written: 12 bytes per (token, head), half read
        and half written) and one moving only its algorithmic bytes (8)."""
        import torch
        w, ssd, dev = self.w, self.ssd, self.dev
        n = w.batch * w.seqlen * w.nheads
        k = max(2, min(64, -(-(1 << 30) // (12 * n))))
        dt0, A, T = self.sets[0]["dt"], self.sets[0]["A"], w.chunk_size
        b, L, H = w.batch, w.seqlen, w.nheads
        sets = [(dt0.clone(), torch.empty(b, H, L, device=dev), torch.empty(b, H, L, device=dev))
                for _ in range(k)]
        for i in range(k):
            ssd.ssd_chunk_cumsum(sets[i][0], A, sets[i][1], sets[i][2], T)
        calls = [lambda s=s: ssd.ssd_chunk_cumsum(s[0], A, s[1], s[2], T) for s in sets]
        out = {"chunk_cumsum": graph_time_ms(calls * max(1, nlaunch // k))}
        del sets
        for key, words in (("copy_same_bytes", 3 * n // 2), ("copy_alg_bytes", n)):
            bufs = [(torch.empty(words, device=dev), torch.empty(words, device=dev))
                    for _ in range(k)]
            calls = [lambda b=b: b[1].copy_(b[0]) for b in bufs]
            for c in calls:
                c()
            out[key] = graph_time_ms(calls * max(1, nlaunch // k))
            del bufs
        return out

    def targets(self, dur: dict) -> dict:
        return _targets(self.w, self.by, dur)

    def summary(self, dur: dict) -> dict:
        """The configs-map entry: tokens/s, per-stage microseconds, HBM
        fractions and the output stage's matrix-core fractions."""
        w = self.w
        kind = mfma_kind(w)
        issued = issued_mfma_flop(w)
        stages = {}
        for n in self.kernels:
            ms = dur[n]
            gbs = self.by[n] / (ms * 1e-3) / 1e9
            e = {"us": round(ms * 1e3, 2), "alg_bytes": self.by[n],
                 "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
            if n in design_extra_bytes(w):
                extra = design_extra_bytes(w)[n]
                e["design_extra_bytes"] = extra
                e["hbm_frac_with_extra"] = round(
                    (self.by[n] + extra) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
            if n == "chunk_cumsum" and "copy_alg_bytes" in dur:
                same, alg = dur["copy_same_bytes"], dur["copy_alg_bytes"]
                e["copy_floor"] = {
                    "same_bytes_us": round(same * 1e3, 2),
                    "alg_bytes_us": round(alg * 1e3, 2),
                    "alg_bytes_hbm_frac": round(
                        self.by[n] / (alg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "note": "device copies over rotating buffers moving the stage's own "
                            "bytes and only its algorithmic bytes: what a kernel with no "
                            "arithmetic reaches at this size"}
            if n in issued:
                peak_tf = BF16_MFMA_TFLOPS if kind[n] == "bf16" else FP32_MFMA_TFLOPS
                tf_alg = self.fl[n] / (ms * 1e-3) / 1e12
                tf_iss = issued[n] / (ms * 1e-3) / 1e12
                e["alg_TFLOP_per_s"] = round(tf_alg, 2)
                e["issued_TFLOP_per_s"] = round(tf_iss, 2)
                e["mfma_instruction"] = kind[n]
                e["mfma_peak_TFLOP_per_s"] = peak_tf
                e["mfma_alg_frac"] = round(tf_alg / peak_tf, 4)
                e["mfma_issued_frac"] = round(tf_iss / peak_tf, 4)
                rec = (committed_profile(w.name, n, "mfma")
                       if n in ("compute_out", "state_and_out") else None)
                if rec is not None:
                    e["mfma_busy_frac_counters"] = round(rec["mfma_busy_frac"], 4)
            stages[n] = e
        step_ms = dur["ssd_forward"]
        step_bytes = sum(self.by[n] for n in self.kernels)
        extra = {}
        if "state_and_out" in self.kernels:
            extra["two_kernel_path_us"] = {n: round(dur[n] * 1e3, 2)
                                           for n in ("fwd_pass_state", "compute_out")}
        return {"north_star_targets": self.targets(dur),
                "shape": {"batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                          "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                          "chunk_size": w.chunk_size, "dtype": w.dtype},
                "tokens_per_s": round(w.tokens / (step_ms * 1e-3), 1),
                "step_us": round(step_ms * 1e3, 2),
                "step_alg_bytes": step_bytes,
                "step_hbm_frac": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                "hbm_floor_us": round(step_bytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2),
                "step_kernels": self.kernels,
                "stages": stages, **extra}


def _targets(w, by, dur) -> dict:
    """The per-stage targets (stage 1 and the state pass at >= 0.6 of the HBM
    peak on their algorithmic bytes; the output stage at >= 40% of the bf16
    matrix peak) against this run's stage kernels, whether or not ssd_forward
    runs stages 2 and 3 fused at this workload.  For the output stage also
    the matrix fraction its issued work would reach if the kernel ran at the
    HBM peak: the most any kernel of that design can show."""
    def hbm(n):
        return by[n] / (dur[n] * 1e-3) / 1e9 / HBM_PEAK_GBS
    issued = issued_mfma_flop(w)["compute_out"]
    # the peak of the instruction the output stage issues (bf16 unless fp32
    # inputs come in 256-token chunks)
    peak = BF16_MFMA_TFLOPS if mfma_kind(w)["compute_out"] == "bf16" else FP32_MFMA_TFLOPS
    a1, a2 = hbm("chunk_cumsum"), hbm("fwd_pass_state")
    iss = issued / (dur["compute_out"] * 1e-3) / 1e12 / peak
    at_peak = issued / (by["compute_out"] / (HBM_PEAK_GBS * 1e9)) / 1e12 / peak
    rec = committed_profile(w.name, "compute_out", "mfma")
    busy = rec["mfma_busy_frac"] if rec is not None else None
    a3 = busy if busy is not None else iss
    return {"a1_chunk_cumsum_hbm_frac": round(a1, 4), "a1_met": a1 >= 0.6,
            "a2_fwd_pass_state_hbm_frac": round(a2, 4), "a2_met": a2 >= 0.6,
            "a3_compute_out_mfma_busy_frac": None if busy is None else round(busy, 4),
            "a3_compute_out_mfma_issued_frac": round(iss, 4),
            "a3_mfma_issued_frac_at_hbm_peak": round(min(1.0, at_peak), 4),
            "a3_met": a3 >= 0.4, "a3_reachable_at_hbm_peak": at_peak >= 0.4,
            "targets": {"a1": "hbm >= 0.6", "a2": "hbm >= 0.6",
                        "a3": f"{mfma_kind(w)['compute_out']} mfma >= 0.4"}}


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


def side_fields(ssd, run, dev, stream, steps, y_dtype, with_gdn):
    """Decode step, conv1d and Gated DeltaNet timings (not part of the step)."""
    import torch
    from ssd_workloads import (GDN_WORKLOADS, conv_workload_for, make_conv_inputs,
                               make_gdn_inputs)
    w, sets, nsets = run.w, run.sets, run.nsets
    b, H, P, N, G = w.batch, w.nheads, w.headdim, w.dstate, w.ngroups
    tin = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    # the streaming decode step at the same batch and heads: one token per
    # sequence from the carried state (read and written in place), replayed
    # from a HIP graph (a step is shorter than one Python launch)
    dec_states = [torch.randn(b, H, P, N, device=dev) for _ in range(nsets)]
    dec_in = [(s["x"][:, 0].contiguous(), s["dt"][:, 0].contiguous(),
               s["B"][:, 0].contiguous(), s["C"][:, 0].contiguous(),
               torch.empty(b, H, P, device=dev, dtype=y_dtype)) for s in sets]

    def dec(i):
        xt, dtt, Bt, Ct, yt = dec_in[i % nsets]
        ssd.ssd_decode_step(xt, dtt, sets[0]["A"], Bt, Ct, sets[0]["D"],
                            dec_states[i % nsets], yt)
    for i in range(5):
        dec(i)
    dec_ms = graph_time_ms([lambda i=i: dec(i) for i in range(50)], nrep=8)
    dec_bytes = (8 * b * H * P * N + (2 if w.dtype == "bf16" else 4) * (b * H * P + 2 * b * G * N)
                 + 4 * b * H + 8 * H + run.y_bytes * b * H * P)
    del dec_states, dec_in

    # the causal depthwise conv1d that feeds this layer's SSD (over the x, B
    # and C channels), x and out in the workload's storage type
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
    conv_ms = graph_time_ms([lambda i=i: ssd.ssd_causal_conv1d(conv_sets[i % nconv][0], cwt,
                                                                cbias, conv_sets[i % nconv][1])
                             for i in range(max(10, nconv))])
    conv_bytes = cset_bytes + 4 * cw.dim * (cw.width + 1)
    del conv_sets, cx0
    out = {
        "decode_step": {"ms": round(dec_ms, 5), "tokens_per_s": round(b / (dec_ms * 1e-3), 1),
                        "alg_bytes": dec_bytes,
                        "GB_per_s": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "note": "one token for each of the batch's sequences, state in place; "
                                "steps replayed from a HIP graph"},
        "causal_conv1d": {"ms": round(conv_ms, 5),
                          "shape": {"batch": cw.batch, "dim": cw.dim, "seqlen": cw.seqlen,
                                    "width": cw.width, "dtype": cw.dtype},
                          "alg_bytes": conv_bytes,
                          "GB_per_s": round(conv_bytes / (conv_ms * 1e-3) / 1e9, 1),
                          "hbm_frac": round(conv_bytes / (conv_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                          "note": "the conv over the layer's x, B, C channels; not part of "
                                  "the step; replayed from a HIP graph"},
    }
    if with_gdn:
        out["gated_deltanet"] = gdn_bench(ssd, GDN_WORKLOADS["gdn_layer_bf16"], make_gdn_inputs,
                                          dev, stream, max(20, steps // 2))
    return out


def bf16_y_entry(ssd, w, dev, nlaunch: int) -> dict:
    """ssd_forward of a bf16 workload writing y in bf16, the output type the
    pages' bf16 problem uses (inputs and outputs bf16, states fp32): tokens/s
    and the step's fraction of 8 TB/s on its algorithmic bytes with 2-byte y.
    The configs entry itself keeps fp32 y."""
    import torch
    r = WorkloadRun(ssd, w, torch.bfloat16, dev)
    for i in range(max(3, r.nsets)):
        r.forward(i)
    ms = graph_time_ms([lambda i=i: r.forward(i) for i in range(nlaunch)])
    step_bytes = sum(r.by[n] for n in r.kernels)
    del r
    return {"tokens_per_s": round(w.tokens / (ms * 1e-3), 1), "step_us": round(ms * 1e3, 2),
            "step_alg_bytes": step_bytes,
            "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_rate(dev) -> float:
    """A 1 GiB device-to-device copy (read + write), timed from a graph of 5
    copies: the runtime's own streaming rate on this GPU, for context."""
    import torch
    csrc = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    ms = graph_time_ms([lambda: cdst.copy_(csrc)] * 5, nrep=1)
    del csrc, cdst
    return 2 * (1 << 28) * 4 / (ms * 1e-3) / 1e9


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wide_fp32")
    ap.add_argument("--y-dtype", default="fp32", choices=["fp32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the named workload (no configs map)")
    ap.add_argument("--no-side", action="store_true",
                    help="skip the decode step, conv1d and Gated DeltaNet timings")
    ap.add_argument("--no-gdn", action="store_true",
                    help="skip the Gated DeltaNet kernels' timing")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter scale)")
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed steps before the warmup steps, until this much time has "
                         "passed (the GPU's clocks reach their steady state)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} "
              "is not supported (the path shards over (batch, head) with no "
              "communication between GPUs).", file=sys.stderr)
        return 2

    import torch

    import mamba_ssd_chunked_fwd_amd as ssd
    from ssd_workloads import WORKLOADS

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ty = torch.bfloat16 if args.y_dtype == "bf16" else torch.float32
    stream = torch.cuda.current_stream(dev)
    nlaunch = max(10, min(40, args.steps // 2))

    run = WorkloadRun(ssd, w, ty, dev)
    # ---- the step: ssd_forward, the whole hot path, as a user calls it.
    # Before the warmup steps, untimed steps until --settle-ms have passed: a
    # few milliseconds of work leave this GPU's clocks ramping, and the steps
    # right after them run about 15% slower than the sustained rate.
    settle_steps, t_settle = 0, time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            run.forward(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - t_settle) * 1e3
    for i in range(args.warmup):
        run.forward(i)
    # the timed steps carry no events between them: nothing but the step's
    # own launches reaches the stream inside the timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run.forward(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dur = run.time_all(nlaunch)
    head = run.summary(dur)
    side = (side_fields(ssd, run, dev, stream, args.steps, ty, not args.no_gdn)
            if not args.no_side else {})
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    copy_gbs = copy_rate(dev)
    inp, nsets, step_flop = run.inp, run.nsets, sum(run.fl[n] for n in run.kernels)
    kernels = run.kernels
    del run
    torch.cuda.empty_cache()

    configs = {}
    if not args.no_configs:
        for name in CONFIG_ORDER:
            if name == w.name:
                configs[name] = head
                continue
            r = WorkloadRun(ssd, WORKLOADS[name], ty, dev)
            configs[name] = r.summary(r.time_all(nlaunch))
            del r
            torch.cuda.empty_cache()
            if WORKLOADS[name].dtype == "bf16" and ty != torch.bfloat16:
                configs[name]["bf16_y"] = bf16_y_entry(ssd, WORKLOADS[name], dev, nlaunch)
                torch.cuda.empty_cache()

    ms_per_step = wall * 1e3 / args.steps
    tokens_per_s = w.tokens / (wall / args.steps)
    stages = head["stages"]
    dom = max(kernels, key=lambda n: stages[n]["us"])
    achieved = stages[dom]["GB_per_s"]
    traffic_rec = committed_profile(w.name, dom, "traffic")
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
        "dtype": "f32" if w.dtype == "fp32" else "bf16",
        "data": "synthetic (seeded; shapes and distributions of the workload)",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen,
                   "nheads": w.nheads, "headdim": w.headdim, "dstate": w.dstate,
                   "ngroups": w.ngroups, "chunk_size": w.chunk_size,
                   "x_dtype": w.dtype, "y_dtype": args.y_dtype,
                   "state_dtype": "fp32", "input_sets_rotated": nsets},
        "roofline": {"bound": "hbm", "kernel": dom,
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (traffic_rec or {}).get("hbm_bytes_per_launch"),
                     "alg_bytes_per_launch": stages[dom]["alg_bytes"],
                     "us_per_launch": stages[dom]["us"]},
        "stages": stages,
        **({"two_kernel_path_us": head["two_kernel_path_us"]}
           if "two_kernel_path_us" in head else {}),
        "settle": {"ms": round(settle_ms, 1), "steps": settle_steps,
                   "note": "untimed steps before the warmup steps, until the GPU's clocks "
                           "settle"},
        "ssd_forward_graph_us": head["step_us"],
        "effective_TFLOP_per_s": round(step_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "hbm_floor_ms": round(head["hbm_floor_us"] / 1e3, 5),
        "copy_GB_per_s_context": round(copy_gbs, 1),
        "configs": configs,
    }
    out.update(side)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
