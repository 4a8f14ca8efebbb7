#!/usr/bin/env python3
"""Throughput benchmark of the Mamba-1 selective-scan forward pass on one
MI355X, on the Mamba-1.4B-shaped workload (batch 8, dim 4096, dstate 16,
seqlen 2048; bf16 u/delta/B/C/z, fp32 A/D/delta_bias/state; softplus with
bias, D skip, silu(z) gate, last_state output).

One step = one ssm_selective_scan_fwd_ws call over the whole batch (inputs
resident in HBM; a workspace only for shapes too small to fill the device,
none at the 1.4B shape).  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--warmup-seconds S] [--gpus 1]
                    [--no-cpu-baseline] [--no-per-call] [--no-ssd] [--calib-copy]
                    [--bwd] [--decode] [--grouped] [--seq-table]

Before the W warm-up steps, calls run untimed for at least S seconds (default
1.0) so that the timed steps see the engine clock at its sustained value.
The line also carries the Mamba-2 chunked scan (SSD) on its workload (batch
4, seqlen 4096, 24 heads, headdim 64, dstate 128, chunk 256, bf16) in "ssd".

Algorithmic HBM bytes per call (inputs read once, outputs written once):
    u, delta, z: 3*b*d*L*es   y: b*d*L*es   B, C: 2*b*N*L*es
    A: 4*d*N   D, delta_bias: 2*4*d   last_state: 4*b*d*N
The roofline is HBM bandwidth: algorithmic bytes per launch / the kernel's
average launch time (HIP events on the launch stream) / 8 TB/s.  The ALU view
is alu_floor: the issue slots the recurrence needs at full VALU rate.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "selective-scan fwd HBM GB/s and % of peak, Mamba-1.4B shape, 1×MI355X"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def mamba1_bytes(b, d, n, L, es):
    return (4 * b * d * L * es + 2 * b * n * L * es + 4 * d * n + 8 * d + 4 * b * d * n)


def ssd_flops(b, L, h, p, n, g, Q):
    """MFMA work of the chunked form: C B^T per (batch, chunk, group) and the
    masked product, chunk states and state-to-output per (batch, chunk, head),
    each counted over the full Q x Q square."""
    nc = math.ceil(L / Q)
    return 2 * b * nc * (g * Q * Q * n + h * Q * Q * p + 2 * h * Q * n * p)


def ssd_bytes(b, L, h, p, n, g):
    """x, dt, B, C read once (bf16), A, D, dt_bias (fp32), y written once
    (bf16) and final_state (fp32)."""
    return 2 * (2 * b * L * h * p + b * L * h + 2 * b * L * g * n) + 3 * 4 * h + 4 * b * h * p * n


# Issue-slot view of the ALU bound.  A wave64 VALU instruction occupies a
# SIMD for 4 cycles (16 lanes per cycle); v_exp_f32 occupies it for two such
# slots.  The recurrence needs at least 4 VALU (delta*A2, delta*u*B, state
# FMA, readout FMA) and one exp per state update: 6 lane-slots.
SLOTS_PER_UPDATE = 6
LANE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9   # CUs x SIMDs x lanes x clock


def alu_floor(updates, kernel_us):
    """Time the state updates alone need at full VALU issue rate, and the
    measured kernel's fraction of it (the per-(b, d, t) work and the readout
    reduce-scatter come on top of this floor)."""
    floor_us = updates * SLOTS_PER_UPDATE / LANE_SLOTS_PER_S * 1e6
    return {"slots_per_update": SLOTS_PER_UPDATE, "floor_us": round(floor_us, 1),
            "frac": round(floor_us / kernel_us, 4)}


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--warmup-seconds", type=float, default=1.0,
                    help="untimed calls for at least this long before the --warmup steps")
    ap.add_argument("--workload", default="m1p4b", choices=["m1p4b", "m130m", "long", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-call", action="store_true",
                    help="skip the per-call flushed timings and the copy bandwidth (for traces)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-ssd", action="store_true", help="leave out the Mamba-2 chunked scan")
    ap.add_argument("--ssd", action="store_true", help=argparse.SUPPRESS)  # (now the default)
    ap.add_argument("--bwd", action="store_true",
                    help="time the backward pass on the same workload also with --no-per-call")
    ap.add_argument("--seq-table", action="store_true",
                    help="also time batch 16, dim 1536, dstate 16, bf16 at seqlen 256..16384")
    ap.add_argument("--grouped", action="store_true",
                    help="also time B, C per group of channels: 8 groups and one per channel")
    ap.add_argument("--spec-point", action="store_true",
                    help="also time the task-spec speed-up point when --no-per-call is given")
    ap.add_argument("--decode", action="store_true",
                    help="also time one decode step (state update) at the same batch/dim/dstate")
    return ap.parse_args()


def calib_copy(torch):
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 5}))


CSRC = os.path.join(ROOT, "mamba_selective_scan_ssm_amd", "csrc")
# The sources each kernel is compiled from (the kernel file and the headers
# it includes), in a fixed order: their combined sha256 ties a committed
# counter summary to the code it was taken on.
KERNEL_SRC = [os.path.join(CSRC, f) for f in
              ("selective_scan.hip", "scan_common.h", "device_math.h", "selective_scan_launch.h")]
SSD_SRC = [os.path.join(CSRC, f) for f in ("ssd_chunk_scan.hip", "device_math.h", "ssd_launch.h")]


def sources_sha256(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        h.update(open(p, "rb").read())
    return h.hexdigest()


def measured_traffic(name: str, srcs, per: str = "launch"):
    """HBM bytes per launch (or per call) from the committed rocprofv3 counter
    summary profiles/<name>_hbm_traffic.md, if it was taken on the kernel
    sources as they are now (else None)."""
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(("#", " ", "|")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    key = f"traffic_bytes_per_{per}"
    if fields.get("kernel_sources_sha256") != sources_sha256(srcs) or key not in fields:
        return None
    return int(fields[key])


def clock_warmup(torch, step, seconds):
    """Untimed calls until at least `seconds` of wall time have passed, so
    that the timed steps run at the sustained engine clock (the first
    launches of a process run while the clock is still ramping up)."""
    calls, t0 = 0, time.perf_counter()
    while True:
        for _ in range(10):
            step()
        calls += 10
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            break
    return {"seconds": round(time.perf_counter() - t0, 3), "calls": calls}


def per_call_flushed(torch, step, calls=50, warm=5):
    """Each call timed on its own with HIP events, after a 1 GiB write that
    evicts the inputs from L2 and the 256 MB MALL (outside the timed span);
    returns median, p10 and p90 in microseconds."""
    import numpy as np
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    for _ in range(warm):
        step()
    times = []
    for _ in range(calls):
        scratch.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    t = np.array(times)
    return {"calls": calls, "l2_mall_flush": "1 GiB write before each call",
            "median_us": round(float(np.median(t)), 2),
            "p10_us": round(float(np.percentile(t, 10)), 2),
            "p90_us": round(float(np.percentile(t, 90)), 2)}


def copy_bandwidth(torch, nbytes=1 << 30, reps=10):
    """Device-to-device copy of 1 GiB: (bytes read + bytes written) / time."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return round(gbs, 1)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity_vs_oracle(got, ref):
    """Errors of the GPU outputs against the oracle's, as the parity tests
    measure them: max |err|, the norm-wise relative error, and the largest
    |err| / (|ref| + rms(ref)) (the bf16 bound is 2e-2 of that)."""
    import numpy as np
    out = {}
    for name, g, r in zip(("y", "last_state"), got, ref):
        err = np.abs(g - r)
        rms = float(np.sqrt(np.mean(r ** 2)))
        out[name] = {"max_abs_err": float(err.max()),
                     "rel_l2": float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)),
                     "max_err_over_abs_ref_plus_rms": float((err / (np.abs(r) + rms)).max())}
    return out


def cpu_baseline(x, cfg, oracle, min_seconds=1.0, gpu_out=None):
    """Time the oracle (as it stands) on the whole workload on the host,
    repeating it until at least `min_seconds` of wall time (about 16 s of CPU
    work on 16 threads).  With gpu_out (y [rows, L], last_state [rows, N] of
    the timed GPU run, float64), also the GPU's errors against the oracle's
    outputs of the same run."""
    threads = oracle.default_threads()
    reps, t0 = 0, time.perf_counter()
    while True:
        ref = oracle.selective_scan(**x, delta_softplus=cfg.softplus, want_y=True,
                                    want_state=True, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    es = 2 if cfg.dtype == "bf16" else 4
    # per-core rate: one thread on the first 256 rows
    rows = list(range(min(256, b * d)))
    t1 = time.perf_counter()
    oracle.selective_scan(**x, delta_softplus=cfg.softplus, rows=rows, nthreads=1)
    one = time.perf_counter() - t1
    parity = parity_vs_oracle(gpu_out, ref) if gpu_out is not None else None
    return {"value": reps * mamba1_bytes(b, d, n, L, es) / dt / 1e9, "unit": "GB/s",
            "cores": threads, "kind": "oracle", "seconds": round(dt, 3), "repetitions": reps,
            "gpu_parity": parity,
            "nproc": os.cpu_count(), "cpu_model": cpu_model(),
            "one_thread_state_updates_per_s": round(len(rows) * L * n / one, 1),
            "sample": f"the whole {cfg.name} workload ({b * d} rows x {L} steps x {n} states, "
                      f"fp64 sequential loop per row, rows over {threads} threads), run {reps}x"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the scan shards over "
              "(batch, channel) rows with no communication, so N GPUs run N independent "
              "copies of this workload.", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.calib_copy:
        calib_copy(torch)
        return

    import mamba_selective_scan_ssm_amd as ssm
    import synth

    ssm.load_library()
    cfg = synth.MAMBA1_CONFIGS[args.workload]
    x = synth.mamba1_inputs(cfg, seed=2)
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    es = 2 if cfg.dtype == "bf16" else 4
    dev = torch.device("cuda:0")
    io = {k: synth.to_device(v, cfg.dtype if k in ("u", "delta", "z", "B", "C") else "f32", dev)
          for k, v in x.items()}
    y = torch.empty_like(io["u"])
    ls = torch.empty((b, d, n), dtype=torch.float32, device=dev)
    handle = ssm.get_handle(0)
    # A workspace only when the rows alone leave the device idle (small
    # batch): then the sequence is also split in time across workgroups.
    ws_bytes = ssm.ssm_selective_scan_fwd_workspace_size(b, d, n, L, handle=handle)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step():
        ssm.ssm_selective_scan_fwd_ws(io["u"], io["delta"], io["A"], io["B"], io["C"], io["D"],
                                      io["z"], io["delta_bias"], cfg.softplus, None, y, ls, ws,
                                      handle=handle)

    # The steps are launched from Python: a cyclic garbage collection in the
    # middle of the timed loop has stalled the launches for tens of
    # milliseconds (seen in kernel traces as one gap between two launches),
    # so the collector runs now and stays off for the GPU measurements.
    gc.collect()
    gc.disable()
    warm = clock_warmup(torch, step, args.warmup_seconds)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    ms_per_step = wall * 1e3 / args.steps
    # the timed run's outputs, for the comparison with the oracle (host copy,
    # outside the timed region)
    gpu_out = None if args.no_cpu_baseline else (
        synth.to_host_f64(y).reshape(b * d, L), synth.to_host_f64(ls).reshape(b * d, n))

    nbytes = mamba1_bytes(b, d, n, L, es)
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    kern_s = ev_ms * 1e-3
    hbm_gbs = nbytes / kern_s / 1e9
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: Mamba-1 selective scan fwd, batch {b}, dim {d}, "
                               f"dstate {n}, seqlen {L}, {cfg.dtype} u/delta/B/C/z, fp32 "
                               "A/D/delta_bias/last_state, softplus(delta+bias), D skip, "
                               "silu(z) gate",
                   "batch": b, "dim": d, "dstate": n, "seqlen": L, "parallelism": "none"},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "elements_per_s": round(b * d * L / (ms_per_step * 1e-3), 1),
        "state_updates_per_s": round(b * d * L * n / (ms_per_step * 1e-3), 1),
        "kernel_avg_us_hip_events": round(ev_ms * 1e3, 3),
        "clock_warmup": warm,
        "time_split_workspace_bytes": ws_bytes,
        "roofline": {"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(hbm_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(f"selective_scan_fwd_kernel_{cfg.name}", KERNEL_SRC),
                     "kernel": "selective_scan_fwd_kernel", "bytes_per_launch": nbytes},
        "alu_floor": alu_floor(b * d * L * n, ev_ms * 1e3),
    }
    if not args.no_per_call:
        out["per_call"] = per_call_flushed(torch, step)
        copy_gbs = copy_bandwidth(torch)
        out["copy_gbs"] = copy_gbs
        out["pct_of_copy"] = round(100.0 * hbm_gbs / copy_gbs, 2)
    if not args.no_ssd:
        out["ssd"] = bench_ssd(args, torch, ssm, synth)
    if args.decode:
        out["decode"] = bench_decode(args, torch, ssm, synth, cfg)
        out["ssd_decode"] = bench_ssd_decode(args, torch, ssm, synth)
    if args.grouped:
        out["grouped"] = [bench_grouped(args, torch, ssm, synth, cfg, io, x, g)
                          for g in (8, d)]
    if args.seq_table:
        out["seq_table"] = bench_seq_table(torch, ssm, synth)
    if args.bwd or not args.no_per_call:
        out["bwd"] = bench_bwd(args, torch, ssm, synth, cfg, io, x)
    if not args.no_per_call or args.spec_point:
        out["spec_point"] = bench_spec_point(torch, ssm, synth)
    if not args.no_cpu_baseline:
        import oracle
        out["cpu_baseline"] = cpu_baseline(x, cfg, oracle, gpu_out=gpu_out)
        out["speedup_vs_oracle"] = round(value / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


def bench_bwd(args, torch, ssm, synth, cfg, io, x):
    """One ssm_selective_scan_bwd call per step (forward recomputed inside,
    every gradient written)."""
    import numpy as np
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    dev = torch.device("cuda:0")
    dy = synth.to_device(np.random.default_rng(11).standard_normal((b, d, L)).astype(np.float32),
                         cfg.dtype, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    du, dd, dz = torch.empty_like(io["u"]), torch.empty_like(io["u"]), torch.empty_like(io["u"])
    dA = torch.empty((d, n), **f32)
    dB, dC = torch.empty((b, n, L), **f32), torch.empty((b, n, L), **f32)
    dD, dbias = torch.empty((d,), **f32), torch.empty((d,), **f32)
    ws = torch.empty(ssm.ssm_selective_scan_bwd_workspace_size(b, d, n, L), dtype=torch.uint8,
                     device=dev)
    handle = ssm.get_handle(0)

    def step():
        ssm.ssm_selective_scan_bwd(io["u"], io["delta"], io["A"], io["B"], io["C"], io["D"],
                                   io["z"], io["delta_bias"], cfg.softplus, None, dy, None, du, dd,
                                   dA, dB, dC, dD, dz, dbias, None, ws, handle=handle)

    steps = max(1, args.steps // 4)
    for _ in range(max(1, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    es = 2 if cfg.dtype == "bf16" else 4
    # inputs u, delta, z, dy and outputs du, ddelta, dz once; B, C in, dB, dC (fp32) out
    nbytes = 7 * b * d * L * es + 2 * b * n * L * es + 2 * b * n * L * 4 + 8 * d * n + 16 * d
    return {"workload": f"{cfg.name} backward: all gradients, forward recomputed inside",
            "ms_per_call": round(ms, 4), "workspace_bytes": ws.numel(),
            "algorithmic_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "state_updates_per_s": round(b * d * L * n / (ms * 1e-3), 1)}


def bench_seq_table(torch, ssm, synth):
    """Batch 16 at seqlen 256, 1024, 4096, 16384 (dim 1536, dstate 16, bf16,
    softplus, D, gate): the shapes of the Blelloch article's V100 timing
    table, whose dim and dstate it does not state (context only)."""
    rows = []
    dev = torch.device("cuda:0")
    for L in (256, 1024, 4096, 16384):
        cfg = synth.Mamba1Config("seq", 16, 1536, 16, L, "bf16", 0.0, 0.5, delta_bias=True,
                                 gate=True, use_D=True)
        x = synth.mamba1_inputs(cfg, seed=8)
        io = {k: synth.to_device(v, "bf16" if k in ("u", "delta", "z", "B", "C") else "f32",
                                 dev) for k, v in x.items()}
        b, d, _ = x["u"].shape
        y = torch.empty_like(io["u"])
        ls = torch.empty((b, d, 16), dtype=torch.float32, device=dev)
        nbytes = ssm.ssm_selective_scan_fwd_workspace_size(b, d, 16, L)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

        def step():
            ssm.ssm_selective_scan_fwd_ws(io["u"], io["delta"], io["A"], io["B"], io["C"],
                                          io["D"], io["z"], io["delta_bias"], True, None, y, ls,
                                          ws)

        for _ in range(5):
            step()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        rows.append({"seqlen": L, "ms_per_call": round(ms, 4),
                     "hbm_gbs": round(mamba1_bytes(b, d, 16, L, 2) / (ms * 1e-3) / 1e9, 1)})
        del io, y, ls, ws
    return rows


def bench_spec_point(torch, ssm, synth):
    """The task-spec page's speed-up point: batch 1, dim 256, seqlen 2048,
    float32, dstate 16 (softplus, D, gate), through ssm_selective_scan_fwd_ws
    (split in time across workgroups at this size)."""
    cfg = synth.Mamba1Config("spec", 1, 256, 16, 2048, "f32", 0.0, 0.5, delta_bias=True,
                             gate=True, use_D=True)
    x = synth.mamba1_inputs(cfg, seed=3)
    dev = torch.device("cuda:0")
    io = {k: synth.to_device(v, "f32", dev) for k, v in x.items()}
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    y = torch.empty_like(io["u"])
    ls = torch.empty((b, d, n), dtype=torch.float32, device=dev)
    nbytes = ssm.ssm_selective_scan_fwd_workspace_size(b, d, n, L)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None

    def step():
        ssm.ssm_selective_scan_fwd_ws(io["u"], io["delta"], io["A"], io["B"], io["C"], io["D"],
                                      io["z"], io["delta_bias"], True, None, y, ls, ws)

    for _ in range(20):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(100):
        step()
    e1.record()
    torch.cuda.synchronize()
    us_host = e0.elapsed_time(e1) / 100 * 1e3
    # The call is a few microseconds of GPU work, of the order of what a
    # Python call costs: 100 calls captured in one HIP graph and replayed
    # give the device time per call.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(100):
            step()
    graph.replay()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 100 * 1e3
    return {"workload": "batch 1, dim 256, seqlen 2048, dstate 16, f32 (task-spec speed-up point)",
            "us_per_call": round(us, 2), "timing": "100 calls in one HIP graph",
            "us_per_call_host_launched": round(us_host, 2), "workspace_bytes": nbytes,
            "hbm_gbs": round(mamba1_bytes(b, d, n, L, 4) / (us * 1e-6) / 1e9, 1)}


def bench_grouped(args, torch, ssm, synth, cfg, io, x, ngroups):
    """ssm_selective_scan_fwd_grouped on the same workload with B, C
    [batch, ngroups, dstate, seqlen] (ngroups = dim: per channel)."""
    import numpy as np
    b, d, L = x["u"].shape
    n = x["A"].shape[1]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(5)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    Bg = torch.randn((b, ngroups, n, L), generator=gen, device=dev).to(dt)
    Cg = torch.randn((b, ngroups, n, L), generator=gen, device=dev).to(dt)
    y = torch.empty_like(io["u"])
    ls = torch.empty((b, d, n), dtype=torch.float32, device=dev)
    handle = ssm.get_handle(0)

    def step():
        ssm.ssm_selective_scan_fwd_grouped(io["u"], io["delta"], io["A"], Bg, Cg, io["D"],
                                           io["z"], io["delta_bias"], cfg.softplus, None, y, ls,
                                           handle=handle)

    steps = max(1, args.steps // 4)
    for _ in range(max(1, args.warmup // 4)):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    es = 2 if cfg.dtype == "bf16" else 4
    nbytes = mamba1_bytes(b, d, n, L, es) + 2 * b * (ngroups - 1) * n * L * es
    gbs = nbytes / (ms * 1e-3) / 1e9
    del Bg, Cg
    return {"workload": f"{cfg.name} with B, C per group: ngroups {ngroups} "
                        f"({d // ngroups} channels each)",
            "ms_per_call": round(ms, 4), "bytes": nbytes, "hbm_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "state_updates_per_s": round(b * d * L * n / (ms * 1e-3), 1)}


def bench_decode(args, torch, ssm, synth, cfg):
    """One ssm_selective_state_update per step over batch x dim rows (state
    read and written in place)."""
    x = synth.mamba1_inputs(cfg, seed=7, seqlen=1)
    b, d, _ = x["u"].shape
    n = x["A"].shape[1]
    dev = torch.device("cuda:0")
    t = {k: synth.to_device(v, cfg.dtype if k in ("u", "delta", "z", "B", "C") else "f32", dev)
         for k, v in x.items()}
    sq = {k: (t[k].reshape(b, -1) if k in ("u", "delta", "z", "B", "C") else t[k]) for k in t}
    state = torch.zeros((b, d, n), dtype=torch.float32, device=dev)
    y = torch.empty_like(sq["u"])
    handle = ssm.get_handle(0)

    def step():
        ssm.ssm_selective_state_update(state, sq["u"], sq["delta"], sq["A"], sq["B"], sq["C"],
                                       sq["D"], sq["z"], sq["delta_bias"], True, y, handle=handle)

    # A step is a few microseconds of GPU work, less than a Python call costs,
    # so the steps are captured once in a HIP graph and replayed.
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    es = 2 if cfg.dtype == "bf16" else 4
    nbytes = 8 * b * d * n + 4 * b * d * es + 2 * b * n * es + 4 * d * n + 8 * d
    return {"workload": f"decode step: batch {b}, dim {d}, dstate {n}, {cfg.dtype}, fp32 state "
                        "updated in place", "timing": f"{args.steps} steps in one HIP graph",
            "us_per_step": round(us, 3),
            "tokens_per_s": round(b / (us * 1e-6), 1),
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes}


def bench_ssd_decode(args, torch, ssm, synth):
    """One ssd_state_update per step at the SSD shape (batch 4, 24 heads,
    headdim 64, dstate 128), state updated in place, steps replayed from a
    HIP graph."""
    import numpy as np
    cfg = synth.SSD_CONFIGS["ssd"]
    s = synth.ssd_inputs(cfg, seed=12, seqlen=1)
    dev = torch.device("cuda:0")
    t = {k: synth.to_device(np.ascontiguousarray(s[k][:, 0]), "bf16", dev)
         for k in ("x", "dt", "B", "C")}
    f = {k: synth.to_device(s[k], "f32", dev) for k in ("A", "D", "dt_bias")}
    b, h, p = t["x"].shape
    n = t["B"].shape[2]
    state = torch.zeros((b, h, p, n), dtype=torch.float32, device=dev)
    y = torch.empty_like(t["x"])
    handle = ssm.get_handle(0)

    def step():
        ssm.ssd_state_update(state, t["x"], t["dt"], f["A"], t["B"], t["C"], f["D"],
                             f["dt_bias"], True, y, handle=handle)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(args.steps):
            step()
    graph.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / args.steps * 1e3
    nbytes = 8 * b * h * p * n + 2 * 2 * b * h * p + 2 * b * h + 2 * 2 * b * n + 12 * h
    return {"workload": f"SSD decode step: batch {b}, heads {h}, headdim {p}, dstate {n}, bf16, "
                        "fp32 state updated in place", "timing": f"{args.steps} steps in one HIP graph",
            "us_per_step": round(us, 3), "tokens_per_s": round(b / (us * 1e-6), 1),
            "hbm_gbs": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": nbytes}


def bench_ssd(args, torch, ssm, synth):
    """The Mamba-2 chunked scan on its workload: ms per call (HIP events over
    the timed calls, after a clock warm-up), MFMA fraction of the bf16 peak,
    and the HBM traffic measured by the committed counter summary."""
    cfg = synth.SSD_CONFIGS["ssd"]
    s = synth.ssd_inputs(cfg, seed=4)
    dev = torch.device("cuda:0")
    t = {k: synth.to_device(v, "bf16" if k in ("x", "dt", "B", "C") else "f32", dev)
         for k, v in s.items()}
    b, L, h, p = s["x"].shape
    n = s["B"].shape[3]
    ws = torch.empty(ssm.ssd_chunk_scan_workspace_size(b, L, h, p, n, cfg.ngroups, cfg.chunk),
                     dtype=torch.uint8, device=dev)
    y = torch.empty_like(t["x"])
    fs = torch.empty((b, h, p, n), dtype=torch.float32, device=dev)

    def step():
        ssm.ssd_chunk_scan_fwd(t["x"], t["dt"], t["A"], t["B"], t["C"], t["D"], t["dt_bias"],
                               True, y, fs, ws, cfg.chunk)

    warm = clock_warmup(torch, step, min(args.warmup_seconds, 0.5))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    per_call = None if args.no_per_call else per_call_flushed(torch, step)
    flops = ssd_flops(b, L, h, p, n, cfg.ngroups, cfg.chunk)
    nbytes = ssd_bytes(b, L, h, p, n, cfg.ngroups)
    tf = flops / (ms * 1e-3) / 1e12
    traffic = measured_traffic("ssd_chunk_scan_ssd", SSD_SRC, per="call")
    return {"workload": f"ssd: Mamba-2 chunked scan, batch {b}, seqlen {L}, heads {h}, "
                        f"headdim {p}, dstate {n}, groups {cfg.ngroups}, chunk {cfg.chunk}, "
                        "bf16 x/dt/B/C/y, fp32 A/D/dt_bias/final_state",
            "ms_per_call": round(ms, 5), "calls": args.steps, "clock_warmup": warm,
            "tokens_per_s": round(b * L / (ms * 1e-3), 1),
            "mfma": {"achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops_per_call": flops},
            "hbm_algorithmic": {"achieved": round(nbytes / (ms * 1e-3) / 1e9, 1),
                                "peak": HBM_PEAK_GBS, "unit": "GB/s", "bytes_per_call": nbytes},
            "traffic": traffic,
            "traffic_over_algorithmic": None if traffic is None else round(traffic / nbytes, 3),
            "per_call": per_call}


if __name__ == "__main__":
    main()
