"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
algorithmic byte counts the roofline divides by.

The byte counts are written out here term by term for the small-model layer
(batch 4, 2048 tokens, 24 heads of 64, state 128, one group, chunk 64, bf16
inputs, fp32 y, no initial state): each stage must move its inputs and
outputs once.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_small_layer():
    import bench
    from ssd_workloads import WORKLOADS
    w = WORKLOADS["small_bf16"]
    b, L, H, P, N, G, T = 4, 2048, 24, 64, 128, 1, 64
    assert (w.batch, w.seqlen, w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk_size) == \
        (b, L, H, P, N, G, T)
    nc = L // T
    x = 2 * b * L * H * P                      # bf16 x
    bc = 2 * b * L * G * N                     # one of B, C (bf16)
    g_dt = 4 * b * L * H * 2                   # g and dt_t (fp32)
    states = 4 * b * H * nc * P * N            # every chunk's starting state (fp32)
    final = 4 * b * H * P * N
    y = 4 * b * L * H * P                      # fp32 y
    by, fl = bench.algorithmic(w, 4)
    # stage 1 reads dt and writes g; its head-major copy of dt is counted
    # apart, as a design choice
    assert by["chunk_cumsum"] == 4 * b * L * H + 4 * b * L * H == 1572864
    assert bench.design_extra_bytes(w)["chunk_cumsum"] == 4 * b * L * H
    assert by["fwd_pass_state"] == x + bc + g_dt + states + final == 132644864
    # stage 3 also reads C and D
    assert by["compute_out"] == x + 2 * bc + g_dt + states + 4 * H + y == 181928032
    # the state pass's contraction: one multiply-add per (token, head, p, n)
    assert fl["fwd_pass_state"] == 2 * b * L * H * P * N


def test_issued_matrix_work_of_the_output_stage():
    """Issued matrix-instruction work of stage 3, from the kernels' block
    structure, for the wide fp32 and the large bf16 layers: never below
    the algorithmic count, and the bf16 form doubles every product with a
    computed operand (hi + lo)."""
    import bench
    from ssd_workloads import WORKLOADS
    for name in ("wide_fp32", "large_bf16", "small_bf16", "long_bf16"):
        w = WORKLOADS[name]
        by, fl = bench.algorithmic(w, 4)
        iss = bench.issued_mfma_flop(w)
        assert iss["compute_out"] >= fl["compute_out"], name
        # bf16: hi + lo of w o x; the wide fp32 layer's stage 2 runs the
        # head-pair kernel on bf16 instructions, six products per product
        assert iss["fwd_pass_state"] == (2 if w.dtype == "bf16" else 6) * fl["fwd_pass_state"]
    # wide fp32 on bf16 instructions (three-term splits, six products):
    # T = 64, 4 row blocks; C S^T 2 T P N per (b, c, h); L'X in 32-token
    # steps, 1 + 1 + 2 + 2 of them over the row blocks; C B^T 10 of 16 blocks
    # once per (b, c, group)
    w = WORKLOADS["wide_fp32"]
    assert bench.mfma_kind(w) == {"fwd_pass_state": "bf16", "compute_out": "bf16",
                                  "state_and_out": "bf16"}
    # the tiny fp32 layer (one head pair) keeps the fp32-instruction state pass
    assert bench.mfma_kind(WORKLOADS["tiny_fp32"])["fwd_pass_state"] == "fp32"
    assert bench.issued_mfma_flop(WORKLOADS["tiny_fp32"])["fwd_pass_state"] == \
        bench.algorithmic(WORKLOADS["tiny_fp32"], 4)[1]["fwd_pass_state"]
    b, H, G, P, N, nc = 64, 48, 8, 64, 64, 16
    per_item = 2 * 64 * P * N + 6 * 32 * 16 * P * 2
    assert bench.issued_mfma_flop(w)["compute_out"] == \
        6 * (b * nc * H * per_item + b * nc * G * 10 * 16 * 16 * N * 2)


def test_fused_pass_accounting_of_the_wide_layer():
    """The wide fp32 layer runs stages 2 and 3 as one kernel: its bytes are
    x, B, C, g and dt_t read once, the states, final state and y written;
    its issued work is C S^T, X^T L'^T and the state update per (b, c, h)
    and C B^T once per (b, c, pair of heads), six bf16 products each."""
    import bench
    from ssd_workloads import WORKLOADS
    w = WORKLOADS["wide_fp32"]
    assert bench.step_kernels(w) == ["chunk_cumsum", "state_and_out"]
    assert bench.step_kernels(WORKLOADS["tiny_fp32"]) == \
        ["chunk_cumsum", "fwd_pass_state", "compute_out"]
    b, L, H, P, N, G, T = 64, 1024, 48, 64, 64, 8, 64
    nc = L // T
    by, fl = bench.algorithmic(w, 4)
    x = 4 * b * L * H * P
    bc = 4 * b * L * G * N
    assert by["state_and_out"] == (x + 2 * bc + 8 * b * L * H + 4 * b * H * nc * P * N
                                   + 4 * b * H * P * N + 4 * H + 4 * b * L * H * P)
    assert fl["state_and_out"] == fl["fwd_pass_state"] + fl["compute_out"]
    per_head = 2 * (2 * T * P * N) + 6 * 32 * 16 * P * 2
    assert bench.issued_mfma_flop(w)["state_and_out"] == \
        6 * (b * nc * H * per_head + b * nc * (H // 2) * 10 * 16 * 16 * N * 2)


def test_bf16_fused_pass_plans_and_accounting():
    """The bf16 layers run stages 2 and 3 as the bf16 fused pass.  On 256
    CUs each chain is cut into a lead run and runs of R chunks, R the chunk
    steps per CU if the walk were spread evenly: small 48 pairs x 32 chunks
    -> R 6, lead 2 + 5 runs of 6; large 80 x 32 -> R 10, lead 2 + 3 runs of
    10; long 16 x 512 -> 16 runs of 32; the run pass walks every run but the
    last.  Issued matrix work per 64-token block of a head: C S^T and the
    update, 2 T P N each with hi + lo, X^T L'^T over six 32-token k-steps
    with hi + lo; C B^T (ten 16x16 blocks) per head pair; the run pass's
    update over the runs before the last."""
    import bench
    from ssd_workloads import WORKLOADS
    plans = {"small_bf16": (6, 6, 2), "large_bf16": (4, 10, 2), "long_bf16": (16, 32, 32)}
    for name, (nr, R, R0) in plans.items():
        w = WORKLOADS[name]
        assert bench.step_kernels(w) == ["chunk_cumsum", "state_and_out"], name
        assert bench.run_plan(w) == {"runs": nr, "run_chunks": R, "lead_chunks": R0,
                                     "run_pass_chunks": w.nchunks - R}, name
        assert R0 + (nr - 1) * R == w.nchunks and 1 <= R0 <= R
    w = WORKLOADS["small_bf16"]
    b, L, H, P, N = 4, 2048, 24, 64, 128
    nblk = L // 64
    per_block = 2 * 2 * (2 * 64 * P * N) + 2 * 6 * 32 * 16 * P * 2
    run_pass = b * H * (32 - 6) * 2 * (2 * 64 * P * N)
    assert bench.issued_mfma_flop(w)["state_and_out"] == \
        b * H * nblk * per_block + b * (H // 2) * nblk * 10 * 16 * 16 * N * 2 + run_pass


def test_north_star_target_summary():
    """The targets object: stage 1 and the state pass against 0.6 of the
    HBM peak on their algorithmic bytes, the output stage against 40% of the
    matrix peak, with the fraction the output stage's issued work would reach
    at the HBM peak (the large layer with fp32 y: 91.8 issued GFLOP over
    690 MB, about 43% of the bf16 peak, so reachable there)."""
    import bench
    from ssd_workloads import WORKLOADS
    w = WORKLOADS["large_bf16"]
    by, _ = bench.algorithmic(w, 4)
    # durations (ms) putting stage 1 at exactly 0.6 and the state pass at 0.3
    dur = {"chunk_cumsum": by["chunk_cumsum"] / (0.6 * 8e12) * 1e3,
           "fwd_pass_state": by["fwd_pass_state"] / (0.3 * 8e12) * 1e3,
           "compute_out": 0.2}
    t = bench._targets(w, by, dur)
    assert abs(t["a1_chunk_cumsum_hbm_frac"] - 0.6) < 1e-3 and t["a1_met"]
    assert abs(t["a2_fwd_pass_state_hbm_frac"] - 0.3) < 1e-3 and not t["a2_met"]
    iss = bench.issued_mfma_flop(w)["compute_out"]
    assert abs(t["a3_compute_out_mfma_issued_frac"] - iss / 0.2e-3 / 2.5e15) < 1e-3
    at_peak = iss / (by["compute_out"] / 8e12) / 2.5e15
    assert 0.4 < at_peak < 0.45
    assert t["a3_reachable_at_hbm_peak"]
    # the small layer's output stage cannot reach 40% even at the HBM peak
    ws = WORKLOADS["small_bf16"]
    bys, _ = bench.algorithmic(ws, 4)
    ts = bench._targets(ws, bys, {k: 1.0 for k in ("chunk_cumsum", "fwd_pass_state",
                                                   "compute_out")})
    assert not ts["a3_reachable_at_hbm_peak"]
