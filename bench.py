"""Benchmark of the chunkwise gated delta rule forward pass on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload main] [--no-cpu-baseline]

A step is one gdn_chunk_fwd call (the whole hot path: decay prefix, Gram and
scores, triangular solve, pseudo-values, output and state scan, all in one
kernel) over the workload's seeded synthetic inputs, already resident in HBM.
For the ``decode`` workload a step is one gdn_recurrent_fwd call (one token
per sequence against a resident state, updated in place).  Prints one JSON line.  ``value`` is
tokens/s = B * T / seconds per step.

roofline: the kernel's algorithmic bytes (read q, k, v, alpha, beta, S0
once; write O and S_final once) divided by its mean launch duration -- the
span of HIP events recorded on the kernel's stream around the K timed
launches, divided by K -- against 8 TB/s HBM.
cpu_baseline: the fp64 CPU oracle timed on this host on a bounded sample of
the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # dense bf16 MFMA
METRIC = "tokens/s and achieved TFLOP/s (% roofline), GDN fwd H=16 T=4096 d=128, 1 MI355X"
# every source file the kernels are built from: traffic figures taken on
# other sources are not reported
KERNEL_SOURCES = sorted(os.path.relpath(os.path.join(dp, f), ROOT)
                        for dp, _, fs in os.walk(os.path.join(ROOT, "gated_delta_rule_13_amd", "csrc"))
                        for f in fs if f.endswith((".h", ".hip")))


def traffic_file(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel sources; else None."""
    try:
        with open(traffic_file(kernel, workload)) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("workload") != workload or rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    """The host CPU's model name (first processor in /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def segments_in_workspace(w, ws_bytes: int, o_bf16: bool) -> int:
    """Segments per sequence of a chunked call, from its workspace size (the
    layout of include/gdn.h: end states and transitions, carried queries,
    then zero-state outputs for bf16 O; 0 bytes: the plain form)."""
    if not ws_bytes:
        return 1
    up = lambda n: (n + 255) // 256 * 256
    bh = w.B * w.H
    rest = bh * w.T * w.dk * 4
    if o_bf16:
        rest = up(rest) + bh * w.T * w.dv * 4
    for nseg in range(2, w.T + 1):
        if up(bh * nseg * (w.dv + w.dk) * w.dk * 4) + rest == ws_bytes:
            return nseg
    raise RuntimeError("workspace size matches no segment count")


def cpu_baseline(x, w, target_seconds=10.0):
    """Time the fp64 oracle on this host over a bounded sample of the same
    workload: whole (b, h) sequences (all of them when the workload is small
    enough, repeated until about ``target_seconds`` have passed), with one
    OpenMP thread per available core up to the number of sequences."""
    import numpy as np
    import oracle

    ncores = len(os.sched_getaffinity(0))
    heads_total = w.B * w.H
    # ~2 GFLOP/s per thread for the plain recurrence (8 d_k d_v flops per head-token)
    per_head_flops = 8.0 * w.dk * w.dv * w.T
    budget_flops = 2.0e9 * min(ncores, heads_total) * target_seconds
    nsel = int(max(1, min(heads_total, budget_flops // per_head_flops)))
    idx = np.linspace(0, heads_total - 1, nsel).round().astype(int)
    pairs = [(int(i) // w.H, int(i) % w.H) for i in idx]
    pick = lambda t: None if t is None else np.stack([t[b, h].double().numpy() for b, h in pairs])[None]
    args = [pick(x["q"]), pick(x["k"]), pick(x["v"]), pick(x["alpha"]), pick(x["beta"])]
    s0 = pick(x["S0"])
    nthreads = min(ncores, nsel)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.recurrent(*args, S0=s0, nthreads=nthreads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_seconds or reps >= 1000:
            break
    head_tokens = nsel * w.T * reps
    # tokens/s on the metric's scale: B*T positions of all H heads per step
    tok_s = head_tokens / dt / w.H
    return {"value": tok_s, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{nsel} of {heads_total} (b,h) sequences at full T={w.T}, "
                      f"{reps} pass(es), fp64 recurrence",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="main")
    ap.add_argument("--o-dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    ap.add_argument("--seg-chunks", type=int, default=0,
                    help="chunks per segment of the sequence-parallel form (gdn_chunk_fwd_seq); "
                         "0: the choice gdn_chunk_fwd makes, a large value: the plain form")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: runs on one GPU only (every (b,h) sequence is independent; "
              "sharding heads over GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import ctypes

    import gated_delta_rule_13_amd as gdn
    from gated_delta_rule_13_amd import _lib
    from gated_delta_rule_13_amd.workloads import (WORKLOADS, algorithmic_bytes,
                                                   algorithmic_flops, make_inputs)

    w = WORKLOADS[args.workload]
    x = make_inputs(w, seed=0)
    dev = torch.device("cuda:0")
    d = {k: (None if x[k] is None else x[k].to(dev)) for k in ("q", "k", "v", "alpha", "beta", "S0")}
    o_dtype = torch.float32 if args.o_dtype == "f32" else torch.bfloat16
    O = torch.empty((w.B, w.H, w.T, w.dv), dtype=o_dtype, device=dev)
    S = torch.empty((w.B, w.H, w.dv, w.dk), dtype=torch.float32, device=dev)

    if args.copy_calibration:
        src = torch.empty(256 * 1024 * 1024, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    recurrent = w.name == "decode"
    if recurrent:
        # a decode step updates the resident state in place
        S.copy_(d["S0"])

    # One call of the binding checks every tensor (and fails loudly on a bad
    # one); the timed steps then call the same C entry point with the
    # arguments marshalled once, so that host overhead stays out of the way
    # of short launches.
    if recurrent:
        gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S,
                              o_dtype=o_dtype, O=O, S_final=S)
    else:
        gdn.gdn_chunk_fwd_seq(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["S0"],
                              chunk_size=w.chunk, seg_chunks=args.seg_chunks, o_dtype=o_dtype,
                              O=O, S_final=S)
    lib = _lib.load()
    ptr = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    shape = gdn.make_shape(w.B, w.H, w.T, w.dk, w.dv, w.chunk, d["q"].dtype, o_dtype)
    sp = ctypes.byref(shape)
    hstream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    # workspace of the sequence-parallel form (none for the plain form)
    ws_bytes = 0 if recurrent else lib.gdn_chunk_fwd_seq_workspace_bytes(sp, args.seg_chunks)
    ws = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=dev) if ws_bytes else None
    ws_ptr = None if ws is None else ctypes.c_void_p((ws.data_ptr() + 255) // 256 * 256)
    if recurrent:
        cargs = (sp, ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]),
                 ptr(S), ptr(O), ptr(S), hstream)
        entry = lib.gdn_recurrent_fwd
    else:
        cargs = (sp, ptr(d["q"]), ptr(d["k"]), ptr(d["v"]), ptr(d["alpha"]), ptr(d["beta"]),
                 ptr(d["S0"]), ptr(O), ptr(S), ws_ptr, ws_bytes, hstream)
        entry = lib.gdn_chunk_fwd
        if args.seg_chunks:
            cargs = (sp, args.seg_chunks) + cargs[1:6] + (None,) + cargs[6:]
            entry = lib.gdn_chunk_fwd_seq

    def step():
        st = entry(*cargs)
        if st != 0:
            _lib.check(st)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: K launches back to back on the kernel's stream, bracketed
    # by one pair of HIP events (the mean launch duration is their span / K).
    stream = torch.cuda.current_stream(dev)
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_begin.record(stream)
    for _ in range(args.steps):
        step()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    mean_kern_s = t_begin.elapsed_time(t_end) / args.steps / 1e3
    ms_per_step = wall / args.steps * 1e3
    # Spread of single launches (a separate, shorter pass with events around
    # each launch; informational only -- the per-launch events add overhead).
    nspread = min(args.steps, 20)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(nspread)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nspread)]
    for i in range(nspread):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    kern_ms = sorted(s_.elapsed_time(e_) for s_, e_ in zip(starts, ends))

    o_bytes = 4 if o_dtype == torch.float32 else 2
    alg_bytes = algorithmic_bytes(w, o_bytes=o_bytes)
    alg_flops = algorithmic_flops(w)
    tokens = w.B * w.T
    value = tokens / (wall / args.steps)
    achieved_gbs = alg_bytes / mean_kern_s / 1e9
    kernel = "gdn_recurrent" if recurrent else "gdn_fwd"
    traffic = (measured_traffic(kernel, w.name)
               if args.o_dtype == "f32" and not args.seg_chunks else None)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "T": w.T, "d_k": w.dk, "d_v": w.dv,
                   "chunk": None if recurrent else w.chunk, "o_dtype": args.o_dtype,
                   "path": "recurrent" if recurrent else "chunked",
                   "segments": None if recurrent else
                   segments_in_workspace(w, ws_bytes, o_dtype != torch.float32),
                   "parallelism": "none (1 GPU)"},
        "head_tokens_per_s": tokens * w.H / (wall / args.steps),
        "tflops": alg_flops / (wall / args.steps) / 1e12,
        "kernel_ms": {"mean": mean_kern_s * 1e3, "single_launch_p10": kern_ms[len(kern_ms) // 10],
                      "single_launch_p50": kern_ms[len(kern_ms) // 2],
                      "single_launch_p90": kern_ms[(9 * len(kern_ms)) // 10]},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes": alg_bytes,
                     "mfma_frac": None if recurrent else
                     alg_flops / mean_kern_s / 1e12 / BF16_PEAK_TFLOPS},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(x, w)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
