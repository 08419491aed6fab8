"""Benchmark of the gfx950 selective scan: one step = one mamba_scan_fwd over one
batch of the Mamba-130M-shaped layer workload (batch 8, 1536 channels,
16 states, 2048 tokens, bf16 inputs, fp32 state, silu gate, last_state
written), inputs already resident in HBM.

Prints one JSON line.  `value` is scan elements (B·D·L·N) per second over the
timed steps.  `roofline` describes the scan kernel: it is bound by vector-ALU
issue (every element needs one v_exp_f32, at a quarter of the fp32 rate, and
four fp32 operations), so the bound reported is "alu" in elements/s, with the
HBM view alongside.  `cpu_baseline` times the fp64 CPU oracle on a bounded
sample of the same workload.  `conv1d` times the causal depthwise Conv1d + SiLU
prologue on the layer's activations against the HBM peak (it is bandwidth
bound).  `backward` times mamba_scan_bwd (the gradients of every input) on the
same workload against its vector-ALU floor.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--decode-steps S]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# Vector-ALU peak of MI355X (gfx950) for this method.  The published fp32 vector
# rate, 157.3 TFLOP/s, is 78.6e12 fp32 lane-operations/s (an FMA counts two flops):
# 256 CUs x 4 SIMDs x 32 lanes x 2.4 GHz, one 64-lane fp32 add/mul/FMA per 2 cycles
# per SIMD.  v_exp_f32 issues at a quarter of that rate (8 lanes per cycle per
# SIMD).  Each scan element needs four fp32 operations (Δ'·A, Δu·B, the state FMA,
# the readout FMA) and one exp: 4/78.6e12 + 1/19.7e12 s, i.e. 9.83e12 elements/s.
# Measured on the chip with a warmed-up clock (2.2-2.4 GHz under load), 8 waves per
# SIMD, register-only loops: VOP2 fp32 instructions 2.6 cycles each, VOP3 v_fma_f32
# 4.4, v_exp_f32 about 10, v_permlane32_swap about 10; the bare recurrence (the
# five instructions per element) 20-22 cycles per 64 elements, about 75 % of this
# peak.
FP32_LANE_OPS = 256 * 4 * 32 * 2.4e9
EXP_LANE_OPS = FP32_LANE_OPS / 4
ALU_PEAK_ELEM = 1.0 / (4.0 / FP32_LANE_OPS + 1.0 / EXP_LANE_OPS)
HBM_PEAK_GBS = 8000.0
# Backward pass, per element: two exps (the forward recompute that writes the
# checkpoints, and the segment recompute) and 21 fp32 operations (4 in each
# recompute; 13 in the adjoint step: λ, the dΔ, dA, dB, du terms, dC, the carry).
BWD_ALU_PEAK_ELEM = 1.0 / (21.0 / FP32_LANE_OPS + 2.0 / EXP_LANE_OPS)


def bwd_algorithmic_bytes(w) -> int:
    """Inputs (and dout) read once, every gradient written once."""
    e = 2 if w.dtype == "bf16" else 4
    K, Bsz, L, Dm, N = w.ndirs, w.batch, w.seqlen, w.dim, w.dstate
    Ku = 1 if w.dir_mode == 3 else K
    act = 2 * (Bsz * Ku * L * Dm + Bsz * K * L * Dm + (Bsz * L * Dm if w.gated else 0)) * e  # u, delta, z and grads
    bc = 2 * 2 * Bsz * K * L * N * e                                                        # B, C and grads
    return act + bc + Bsz * L * Dm * e + 2 * (K * Dm * N * 4 + 2 * K * Dm * 4)             # dout; A, D, bias, grads


def algorithmic_bytes(w) -> int:
    """Each input read once, each output written once (bf16 = 2 B; A, D, bias, state = 4 B)."""
    e = 2 if w.dtype == "bf16" else 4
    K, Bsz, L, Dm, N = w.ndirs, w.batch, w.seqlen, w.dim, w.dstate
    Ku = 1 if w.dir_mode == 3 else K
    by = Bsz * Ku * L * Dm * e          # u
    by += Bsz * K * L * Dm * e          # delta
    by += (Bsz * L * Dm * e) if w.gated else 0  # z
    by += 2 * Bsz * K * L * N * e       # B, C
    by += Bsz * L * Dm * e              # out
    by += Bsz * K * Dm * N * 4          # last_state
    by += K * Dm * N * 4 + 2 * K * Dm * 4  # A, D, delta_bias
    return by


def source_hash() -> str:
    """Hash of the library's code with comments and blank space removed, so a
    counter summary stays valid across comment-only edits."""
    h = hashlib.sha256()
    for f in ("include/mamba_scan.h", "selective_state_space_mamba_amd/csrc/mamba_scan.hip",
              "selective_state_space_mamba_amd/csrc/scan_inst.hip",
              "selective_state_space_mamba_amd/csrc/row_inst.hip",
              "selective_state_space_mamba_amd/csrc/scan_launch.h",
              "selective_state_space_mamba_amd/csrc/scan_kernels.h",
              "selective_state_space_mamba_amd/csrc/scan_row.h",
              "selective_state_space_mamba_amd/csrc/device_math.h",
              "selective_state_space_mamba_amd/build.py"):
        with open(os.path.join(ROOT, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes from the committed rocprofv3 counter summary
    (profiles/scan_fwd_<workload>_counters.md), if it was taken on the current
    kernel sources; else None.  key: hbm_bytes_per_launch (the scan kernel's
    output launch) or hbm_bytes_per_call (every kernel of one forward call)."""
    path = os.path.join(ROOT, "profiles", "scan_fwd_%s_counters.md" % workload)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            parts = line.strip().split(":", 1)
            if len(parts) == 2 and parts[0] in ("source_hash", key):
                rec[parts[0]] = parts[1].strip()
    if rec.get("source_hash") != source_hash() or key not in rec:
        return None
    return int(rec[key])


def cpu_baseline(w, x=None, budget_s: float = 15.0, sample_note: str = ""):
    """Time the fp64 oracle on a bounded sample of the workload's (b, d) rows
    (drawn without replacement).  x: host inputs of w (make_inputs layout);
    drawn here when None.  w.dim may be a channel subset of the named workload
    (sample_note says which)."""
    import oracle
    from selective_state_space_mamba_amd import inputs as I
    if x is None:
        x = I.make_inputs(w)
    threads = min(16, os.cpu_count() or 1)
    rng = np.random.Generator(np.random.PCG64(3))
    total = w.batch * w.dim

    def pick(n):
        flat = np.sort(rng.choice(total, size=min(n, total), replace=False))
        return np.stack([flat // w.dim, flat % w.dim], axis=1).astype(np.int64)

    def run(r, nthreads):
        oracle.scan(x["u"], x["delta"], x["A"], x["B"], x["C"], x["D"], x["z"], x["delta_bias"],
                    dir_mode=w.dir_mode, height=w.height, width=w.width, rows=r, nthreads=nthreads)
    # calibrate on a few rows, then size the sample to about budget_s / 3 per pass
    cal = pick(min(64, total))
    t0 = time.perf_counter()
    run(cal, threads)
    per_row = (time.perf_counter() - t0) / len(cal)
    n = int(min(total, max(len(cal), budget_s / 3 / max(per_row, 1e-9))))
    rows = pick(n)
    # passes over the sample until about budget_s / 3 seconds (a sample that
    # is the whole workload may take well under a second)
    t0 = time.perf_counter()
    passes = 0
    while True:
        run(rows, threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= budget_s / 3 or passes >= 100:
            break
    el = passes * n * w.ndirs * w.seqlen * w.dstate
    # one thread, on the first rows of the sample, about budget_s / 5 seconds
    n1 = int(min(n, max(1, budget_s / 5 / max(per_row * threads, 1e-9))))
    t0 = time.perf_counter()
    run(rows[:n1], 1)
    dt1 = time.perf_counter() - t0
    el1 = n1 * w.ndirs * w.seqlen * w.dstate
    return {"value": el / dt, "unit": "scan elements/s", "cores": threads, "kind": "oracle",
            "sample": "%d distinct (b, d) rows of %d%s of %s, all %d tokens, %d states and %d directions, fp64, "
                      "%d passes in %.1f s" % (n, total, sample_note, w.name, w.seqlen, w.dstate, w.ndirs, passes, dt),
            "nproc": os.cpu_count(),
            "single_thread": {"value": el1 / dt1, "unit": "scan elements/s",
                              "sample": "%d of those rows, %.1f s" % (n1, dt1)}}


def decode_cpu_baseline(x, steps: int, budget_s: float = 3.0):
    """Time the oracle's one-token step over every (b, d) row (single thread)."""
    import oracle
    st = np.zeros((x["B"].shape[0], x["A"].shape[-2], x["A"].shape[-1]), dtype=np.float64)
    t0 = time.perf_counter()
    done = 0
    while done < steps:
        oracle.step(st, x["u"][:, done], x["delta"][:, done], x["A"], x["B"][:, done], x["C"][:, done], x["D"],
                    None if x["z"] is None else x["z"][:, done], x["delta_bias"])
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"us_per_step": dt * 1e6 / done, "steps": done, "cores": 1, "kind": "oracle",
            "sample": "%d steps over all %d (b, d) rows, fp64" % (done, st.shape[0] * st.shape[1])}


def timed_region(torch, stream, fn, n):
    """n back-to-back calls with one HIP event pair on the launch stream
    around all of them (no event between calls: an event packet between two
    kernels delays the second by a few microseconds).  Returns (wall seconds
    from synchronisation to synchronisation, GPU ms per call)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(n):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return time.perf_counter() - t0, e0.elapsed_time(e1) / n


def per_call_ms(torch, stream, fn, n):
    """Durations of n calls, each between its own HIP event pair (for the
    median and minimum; each interval also holds the event's own latency)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(stream)
        fn(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def warm_up(torch, stream, fn, min_calls: int, min_gpu_ms: float):
    """At least min_calls calls, and more until min_gpu_ms of GPU time has run
    (the clocks need some tens of milliseconds of work to settle).  Returns
    (calls, gpu_ms)."""
    calls, gpu_ms = 0, 0.0
    while calls < min_calls or gpu_ms < min_gpu_ms:
        n = max(1, min_calls - calls) if calls < min_calls else max(1, calls // 2)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(calls + i)
        e1.record(stream)
        torch.cuda.synchronize()
        gpu_ms += e0.elapsed_time(e1)
        calls += n
        if calls > 100000:
            break
    return calls, gpu_ms


def copy_ceiling(torch, stream, nbytes: int, reps: int = 10):
    """Rate of torch's device copy moving `nbytes` per call (nbytes/2 read and
    nbytes/2 written), over three rotating buffer pairs so that the 256 MB
    Infinity Cache cannot serve it."""
    half = max(1 << 20, nbytes // 2) // 16 * 16
    pairs = [(torch.empty(half, dtype=torch.uint8, device="cuda:0"),
              torch.empty(half, dtype=torch.uint8, device="cuda:0")) for _ in range(3)]
    for a, b in pairs:
        a.fill_(1)
    with torch.cuda.stream(stream):
        for i in range(6):
            pairs[i % 3][1].copy_(pairs[i % 3][0])
        _, ms = timed_region(torch, stream, lambda i: pairs[i % 3][1].copy_(pairs[i % 3][0]), reps)
    del pairs
    s = ms * 1e-3
    return {"op": "torch device copy, %d bytes read + %d written per call" % (half, half),
            "us_per_call": s * 1e6, "gbs": 2 * half / s / 1e9, "frac_of_peak": 2 * half / s / 1e9 / HBM_PEAK_GBS}


def time_config(torch, ms, I, w, steps: int, warm_ms: float, stream, cpu: bool):
    """One forward workload at full size: inputs drawn on the GPU (enough sets
    to exceed the Infinity Cache), HIP-event timing of back-to-back calls after
    a warm-up of at least warm_ms of GPU time, the rooflines, a copy ceiling of the same
    byte count, and the oracle on a channel sample."""
    dev = torch.device("cuda:0")
    alg = algorithmic_bytes(w)
    nsets = max(1, min(3, -(-600_000_000 // alg)))
    sets = [I.make_inputs_device(w, dev, seed=w.seed + 1000 * s_) for s_ in range(nsets)]
    K = w.ndirs
    kx = () if K == 1 else (K,)
    outs = [torch.empty((w.batch, w.seqlen, w.dim), dtype=sets[0]["u"].dtype, device=dev) for _ in sets]
    states = [torch.empty((w.batch,) + kx + (w.dim, w.dstate), dtype=torch.float32, device=dev) for _ in sets]
    dims = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_BF16 if w.dtype == "bf16" else ms.DTYPE_F32,
                        height=w.height, width=w.width)
    ws = torch.empty(max(ms.workspace_bytes(dims, w.dir_mode), 256), dtype=torch.uint8, device=dev)

    def step(i):
        s_ = sets[i % nsets]
        ms.scan_fwd(s_["u"], s_["delta"], s_["A"], s_["B"], s_["C"], s_["D"], s_["z"], s_["delta_bias"],
                    dir_mode=w.dir_mode, height=w.height, width=w.width, out=outs[i % nsets],
                    last_state=states[i % nsets], workspace=ws, stream=stream)
    with torch.cuda.stream(stream):
        wcalls, wms = warm_up(torch, stream, step, 2, warm_ms)
        _, region_ms = timed_region(torch, stream, step, steps)
        launch_ms = per_call_ms(torch, stream, step, steps)
    avg = region_ms * 1e-3
    el = w.elements
    rec = {"config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                      "dir_mode": ["fwd", "bwd", "bidir", "cross2d"][w.dir_mode], "gated": w.gated,
                      "height": w.height, "width": w.width, "dtype": w.dtype},
           "calls": steps, "input_sets": nsets, "warmup_calls": wcalls, "warmup_gpu_ms": wms,
           "us_per_call": avg * 1e6, "median_us": float(np.median(launch_ms)) * 1e3,
           "min_us": float(np.min(launch_ms)) * 1e3, "elements": el, "elements_per_s": el / avg,
           "alu_frac": el / avg / ALU_PEAK_ELEM, "algorithmic_bytes": alg, "hbm_gbs": alg / avg / 1e9,
           "hbm_frac": alg / avg / 1e9 / HBM_PEAK_GBS, "workspace_bytes": int(ws.numel()),
           "traffic": measured_traffic(w.name, "hbm_bytes_per_call"),
           "traffic_unit": "HBM bytes per forward call, every kernel of it (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)"}
    rec["copy_ceiling"] = copy_ceiling(torch, stream, alg)
    if cpu:
        # a channel sample: every batch, direction and token of 2 to 256 channels,
        # about a million oracle rows x tokens at most
        nch = int(max(2, min(256, w.dim, 4_000_000 // max(1, w.batch * w.seqlen))))
        chans = np.sort(np.random.Generator(np.random.PCG64(5)).choice(w.dim, size=nch, replace=False))
        xs = I.host_channel_sample(w, sets[0], chans)
        rec["cpu_baseline"] = cpu_baseline(w.with_(dim=nch), xs, budget_s=9.0,
                                           sample_note=" (channels %s of %d, drawn on the GPU)"
                                           % (_span(chans), w.dim))
    del sets, outs, states, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def _span(ch):
    return "%d..%d, %d of them" % (int(ch[0]), int(ch[-1]), len(ch))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # the GPU needs some tens of milliseconds of work before its clocks settle:
    # after 5 warm-up calls (~1 ms) the next 50 forward calls of the 130M layer
    # ran 7 % slower than the 50 after them
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warmup-ms", type=float, default=250.0,
                    help="keep warming up until this much GPU time has run, whatever --warmup says")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="timed calls of each of the other specified workloads (0: skip them)")
    ap.add_argument("--workload", default="mamba130m_layer")
    ap.add_argument("--sets", type=int, default=3, help="input sets rotated between steps (defeats the 256 MB MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=512)
    ap.add_argument("--conv-steps", type=int, default=20, help="timed calls of the Conv1d + SiLU prologue (0: skip)")
    ap.add_argument("--bwd-steps", type=int, default=10, help="timed calls of the backward pass (0: skip)")
    ap.add_argument("--variant-steps", type=int, default=20,
                    help="timed calls of each forward option (exact ZOH, initial state; 0: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the timed region, run one torch elementwise kernel that reads and writes a "
                         "MIB-MiB buffer (known bytes, used to scale rocprofv3 FETCH_SIZE / WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the scan library has no multi-GPU path (its (direction, "
              "batch, channel) rows would shard across GPUs with no communication)", file=sys.stderr)
        sys.exit(2)

    import torch
    import selective_state_space_mamba_amd as ms
    from selective_state_space_mamba_amd import inputs as I

    ms.load_library()
    w = I.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream()

    def todev(v):
        if v is None:
            return None
        if v.dtype == np.uint16:
            return torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(v)).to(dev)

    sets = []
    host0 = None
    for s in range(args.sets):
        x = I.make_inputs(w.with_(seed=w.seed + 1000 * s))
        if s == 0:
            host0 = x
        sets.append({k: todev(v) for k, v in x.items()})
    K = w.ndirs
    kx = () if K == 1 else (K,)
    outs = [torch.empty((w.batch, w.seqlen, w.dim), dtype=sets[0]["u"].dtype, device=dev) for _ in sets]
    states = [torch.empty((w.batch,) + kx + (w.dim, w.dstate), dtype=torch.float32, device=dev) for _ in sets]
    dims = ms.make_dims(w.batch, w.dim, w.seqlen, w.dstate, ms.DTYPE_BF16 if w.dtype == "bf16" else ms.DTYPE_F32,
                        height=w.height, width=w.width)
    ws_bytes = ms.workspace_bytes(dims, w.dir_mode)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % len(sets)]
        ms.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"],
                    dir_mode=w.dir_mode, height=w.height, width=w.width, out=outs[i % len(sets)],
                    last_state=states[i % len(sets)], workspace=ws, stream=stream)

    with torch.cuda.stream(stream):
        # the W warm-up calls asked for, and more until the GPU has run at
        # least --warmup-ms of this work (its clocks settle after some tens of
        # milliseconds)
        warm_calls, warm_ms = warm_up(torch, stream, step, args.warmup, args.warmup_ms)
        torch.cuda.synchronize()
        # timed region: exactly K steps, wall clock around synchronisations
        # and one HIP event pair on the launch stream around the K launches
        wall, region_ms = timed_region(torch, stream, step, args.steps)
        # then K more, each between its own event pair (median, minimum)
        launch_ms = per_call_ms(torch, stream, step, args.steps)

    ms_step = wall * 1e3 / args.steps
    el = w.elements
    value = el / (wall / args.steps)
    avg_launch_s = region_ms * 1e-3
    alg_bytes = algorithmic_bytes(w)
    ach_elem = el / avg_launch_s / 1e9
    hbm_gbs = alg_bytes / avg_launch_s / 1e9
    traffic = measured_traffic(w.name)

    decode = None
    if args.decode_steps > 0 and w.dir_mode == 0:
        s0 = sets[0]
        st = states[0].clone()
        ut = s0["u"][:, -1].contiguous()
        dt_ = s0["delta"][:, -1].contiguous()
        Bt = s0["B"][:, -1].contiguous()
        Ct = s0["C"][:, -1].contiguous()
        zt = s0["z"][:, -1].contiguous() if s0["z"] is not None else None
        o = torch.empty_like(ut)
        with torch.cuda.stream(stream):
            for _ in range(10):
                ms.scan_step(st, ut, dt_, s0["A"], Bt, Ct, s0["D"], zt, s0["delta_bias"], out=o, stream=stream)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.decode_steps):
                ms.scan_step(st, ut, dt_, s0["A"], Bt, Ct, s0["D"], zt, s0["delta_bias"], out=o, stream=stream)
            torch.cuda.synchronize()
            dec_s = time.perf_counter() - t0
            # the same loop through a ScanStepper (fixed operands checked once)
            stepper = ms.ScanStepper(st, s0["A"], s0["D"], s0["delta_bias"], dtype=ut.dtype, stream=stream)
            for _ in range(10):
                stepper(ut, dt_, Bt, Ct, zt, out=o)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.decode_steps):
                stepper(ut, dt_, Bt, Ct, zt, out=o)
            torch.cuda.synchronize()
            sdec_s = time.perf_counter() - t0
            # and with static per-token buffers bound once (one C call per step)
            stepper.bind(ut, dt_, Bt, Ct, zt, out=o)
            for _ in range(10):
                stepper.step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.decode_steps):
                stepper.step()
            torch.cuda.synchronize()
            bdec_s = time.perf_counter() - t0
        # the same loop captured once as a HIP graph and replayed (no host
        # work per step): the kernel-bound rate of the decode loop
        graph = torch.cuda.CUDAGraph()
        cs = torch.cuda.Stream()
        cs.wait_stream(stream)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cs):
            for _ in range(args.decode_steps):
                ms.scan_step(st, ut, dt_, s0["A"], Bt, Ct, s0["D"], zt, s0["delta_bias"], out=o, stream=cs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        gdec_s = time.perf_counter() - t0
        del graph
        decode = {"steps": args.decode_steps, "us_per_step": dec_s * 1e6 / args.decode_steps,
                  "stepper_us_per_step": sdec_s * 1e6 / args.decode_steps,
                  "bound_stepper_us_per_step": bdec_s * 1e6 / args.decode_steps,
                  "graph_us_per_step": gdec_s * 1e6 / args.decode_steps,
                  "state_bytes_per_step": 2 * w.batch * w.dim * w.dstate * 4,
                  "elements_per_step": w.batch * w.dim * w.dstate,
                  "cpu_baseline": None if args.no_cpu_baseline else decode_cpu_baseline(host0, args.decode_steps)}

    conv = None
    if args.conv_steps > 0 and w.dir_mode == 0:
        W = 4
        cxs = [{k: todev(v) for k, v in I.make_conv_inputs(w.batch, w.seqlen, w.dim, W, w.dtype,
                                                           w.seed + 77 + s_).items()} for s_ in range(len(sets))]
        couts = [torch.empty_like(c["x"]) for c in cxs]
        with torch.cuda.stream(stream):
            for i in range(3):
                ms.conv1d_silu(cxs[i % len(cxs)]["x"], cxs[i % len(cxs)]["weight"], cxs[i % len(cxs)]["bias"],
                               out=couts[i % len(cxs)], stream=stream)
            torch.cuda.synchronize()
            def cstep(i):
                c = cxs[i % len(cxs)]
                ms.conv1d_silu(c["x"], c["weight"], c["bias"], out=couts[i % len(cxs)], stream=stream)
            _, conv_ms = timed_region(torch, stream, cstep, args.conv_steps)
        conv_s = conv_ms * 1e-3
        e = 2 if w.dtype == "bf16" else 4
        cbytes = 2 * w.batch * w.seqlen * w.dim * e + w.dim * (W + 1) * 4
        conv = {"op": "causal depthwise Conv1d (%d taps) + SiLU, [B][L][D] = [%d][%d][%d] %s"
                      % (W, w.batch, w.seqlen, w.dim, w.dtype),
                "us_per_call": conv_s * 1e6, "algorithmic_bytes": cbytes, "achieved_gbs": cbytes / conv_s / 1e9,
                "peak_gbs": HBM_PEAK_GBS, "frac": cbytes / conv_s / 1e9 / HBM_PEAK_GBS, "bound": "hbm"}

    variants = None
    if args.variant_steps > 0:
        # the forward options on the same inputs, timed like the plain forward
        # (HIP events on the launch stream around each call)
        inits = [torch.randn(st.shape, dtype=torch.float32, device=dev, generator=torch.Generator(dev).manual_seed(7 + j))
                 for j, st in enumerate(states)]

        def vstep(i, **kw):
            s = sets[i % len(sets)]
            ms.scan_fwd(s["u"], s["delta"], s["A"], s["B"], s["C"], s["D"], s["z"], s["delta_bias"],
                        dir_mode=w.dir_mode, height=w.height, width=w.width, out=outs[i % len(sets)],
                        last_state=states[i % len(sets)], workspace=ws, stream=stream, **kw)

        # the three calls interleaved, so that each sees the same clocks
        fns = [vstep, lambda i: vstep(i, exact_zoh=True), lambda i: vstep(i, initial_state=inits[i % len(inits)])]
        with torch.cuda.stream(stream):
            for i in range(20):
                for fn in fns:
                    fn(i)
            torch.cuda.synchronize()
            evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
                   for _ in range(args.variant_steps)]
            for i in range(args.variant_steps):
                for j, fn in enumerate(fns):
                    evs[i][j][0].record(stream)
                    fn(i)
                    evs[i][j][1].record(stream)
            torch.cuda.synchronize()
        plain_s, exact_s, init_s = (float(np.mean([e[j][0].elapsed_time(e[j][1]) for e in evs])) * 1e-3
                                    for j in range(len(fns)))
        variants = {"plain_us_per_call": plain_s * 1e6,
                    "exact_zoh": {"op": "forward with the exact zero-order hold for the input term",
                                  "us_per_call": exact_s * 1e6, "elements_per_s": el / exact_s,
                                  "vs_plain": exact_s / plain_s},
                    "initial_state": {"op": "forward resumed from a given [B][K][D][N] float32 state",
                                      "us_per_call": init_s * 1e6, "elements_per_s": el / init_s,
                                      "vs_plain": init_s / plain_s}}
        del inits

    bwd = None
    if args.bwd_steps > 0 and w.dstate <= 16:
        douts = [todev(I.make_dout(w.with_(seed=w.seed + 1000 * s_))) for s_ in range(len(sets))]
        bws = torch.empty(ms.bwd_workspace_bytes(dims, w.dir_mode), dtype=torch.uint8, device=dev)

        def bstep(i):
            s_ = sets[i % len(sets)]
            return ms.scan_bwd(s_["u"], s_["delta"], s_["A"], s_["B"], s_["C"], s_["D"], s_["z"], s_["delta_bias"],
                               dout=douts[i % len(sets)], dir_mode=w.dir_mode, height=w.height, width=w.width,
                               workspace=bws, stream=stream)
        with torch.cuda.stream(stream):
            # the inputs above took the host a while, and an idle GPU's clocks
            # drop: warm up for --warmup-ms of backward work as for the forward
            bwarm_calls, bwarm_ms = warm_up(torch, stream, bstep, 3, args.warmup_ms)
            _, bwd_ms = timed_region(torch, stream, bstep, args.bwd_steps)
        bwd_s = bwd_ms * 1e-3
        # the training pass with a saved forward state: mamba_scan_fwd_save,
        # then mamba_scan_bwd reading it instead of recomputing the states
        sbytes = ms.saved_bytes(dims, w.dir_mode, w.gated)
        saveds = [torch.empty(sbytes, dtype=torch.uint8, device=dev) for _ in sets]

        def fsave(i):
            s_ = sets[i % len(sets)]
            ms.scan_fwd_save(s_["u"], s_["delta"], s_["A"], s_["B"], s_["C"], s_["D"], s_["z"], s_["delta_bias"],
                             dir_mode=w.dir_mode, height=w.height, width=w.width, out=outs[i % len(sets)],
                             last_state=states[i % len(sets)], workspace=ws, saved=saveds[i % len(sets)],
                             stream=stream)

        def bsaved(i):
            s_ = sets[i % len(sets)]
            return ms.scan_bwd(s_["u"], s_["delta"], s_["A"], s_["B"], s_["C"], s_["D"], s_["z"], s_["delta_bias"],
                               dout=douts[i % len(sets)], dir_mode=w.dir_mode, height=w.height, width=w.width,
                               workspace=bws, saved=saveds[i % len(sets)], stream=stream)
        with torch.cuda.stream(stream):
            for i in range(3):
                fsave(i)
                bsaved(i)
            torch.cuda.synchronize()
            fev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.bwd_steps)]
            bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(args.bwd_steps)]
            for i in range(args.bwd_steps):
                fev[i][0].record(stream)
                fsave(i)
                fev[i][1].record(stream)
                bev[i][0].record(stream)
                bsaved(i)
                bev[i][1].record(stream)
            torch.cuda.synchronize()
        fsave_s = float(np.mean([a.elapsed_time(b) for a, b in fev])) * 1e-3
        bsaved_s = float(np.mean([a.elapsed_time(b) for a, b in bev])) * 1e-3
        bbytes = bwd_algorithmic_bytes(w)
        bwd = {"op": "mamba_scan_bwd: gradients of u, delta, A, B, C, D, z, delta_bias, initial state",
               "us_per_call": bwd_s * 1e6, "elements_per_s": el / bwd_s, "bound": "alu",
               "peak_elements_per_s": BWD_ALU_PEAK_ELEM, "frac": el / bwd_s / BWD_ALU_PEAK_ELEM,
               "algorithmic_bytes": bbytes, "hbm_gbs": bbytes / bwd_s / 1e9,
               "workspace_bytes": int(bws.numel()), "warmup_calls": bwarm_calls, "warmup_gpu_ms": bwarm_ms,
               "saved_state": {"op": "mamba_scan_fwd_save, then mamba_scan_bwd from its saved state (no recompute)",
                               "bytes": int(sbytes), "fwd_save_us_per_call": fsave_s * 1e6,
                               "bwd_us_per_call": bsaved_s * 1e6,
                               "fwd_plus_bwd_us": (fsave_s + bsaved_s) * 1e6,
                               "fwd_plus_recomputing_bwd_us": (avg_launch_s + bwd_s) * 1e6}}
        del bws, douts, saveds

    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 2.0, out=dst)  # one elementwise kernel: reads and writes MIB MiB
        torch.cuda.synchronize()
        del src, dst

    copy = copy_ceiling(torch, stream, alg_bytes)
    del sets, outs, states, ws
    torch.cuda.empty_cache()
    configs = {}
    if args.config_steps > 0:
        for name in ("long_context", "vim_bidir_224", "vim_bidir_1248", "vmamba_ss2d"):
            if name == w.name:
                continue
            wc = I.WORKLOADS[name]
            print("[bench] %s" % name, file=sys.stderr, flush=True)
            configs[name] = time_config(torch, ms, I, wc, max(5, args.config_steps if name != "long_context"
                                                              else args.config_steps // 4),
                                        args.warmup_ms, stream, not args.no_cpu_baseline)
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, host0)
    rec = {
        "metric": "scan elements (B*D*L*N)/s, selective scan forward, bf16 L=2048 D=1536 N=16",
        "value": value,
        "unit": "elements/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_calls_run": warm_calls,
        "warmup_gpu_ms": warm_ms,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic (seeded N(0,1) inputs, S4D-real A, %d input sets rotated)" % args.sets,
        "config": {"workload": w.name, "batch": w.batch, "dim": w.dim, "seqlen": w.seqlen, "dstate": w.dstate,
                   "dir_mode": ["fwd", "bwd", "bidir", "cross2d"][w.dir_mode], "gated": w.gated,
                   "state_dtype": "f32", "parallelism": "single GPU"},
        "roofline": {"bound": "alu", "achieved": ach_elem, "peak": ALU_PEAK_ELEM / 1e9, "unit": "Gelem/s",
                     "frac": ach_elem / (ALU_PEAK_ELEM / 1e9), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE)",
                     "traffic_gbs": (traffic / avg_launch_s / 1e9) if traffic else None,
                     "kernel_avg_us": avg_launch_s * 1e6,
                     "kernel_median_us": float(np.median(launch_ms)) * 1e3,
                     "kernel_min_us": float(np.min(launch_ms)) * 1e3,
                     "hbm": {"achieved": hbm_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": hbm_gbs / HBM_PEAK_GBS,
                             "algorithmic_bytes": alg_bytes, "copy_ceiling": copy}},
        "cpu_baseline": cpu,
        "decode": decode,
        "conv1d": conv,
        "backward": bwd,
        "variants": variants,
        "configs": configs,
        "source_hash": source_hash(),
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
