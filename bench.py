"""Benchmark of the verification step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--mode stochastic]

A step is one sv_verify_* call over one batch of synthetic inputs already
resident in HBM: every row of the hot path (row statistics over all logits,
acceptance ratios, accept-prefix scan, corrective/bonus draw, outputs; plus
candidate selection for the multi-candidate workload).  The default workload
is B=256 sequences, k=8 draft tokens, V=128256, bfloat16 logits, stochastic
mode.  Prints one JSON line.

Other modes, for the profiler:
  --copy-calibration   time a plain device-to-device copy of 1 GiB (the
                       reference kernel for HBM byte counters)
  --no-cpu-baseline    skip the CPU oracle timing
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

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
KERNEL_SRC = os.path.join(ROOT, "draft_token_verification_10_amd", "csrc", "sv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def algorithmic_bytes(spec, mode: str) -> int:
    """Bytes the method itself must move per call: every logit row once, the
    draft tokens and uniforms in, accept_len and tokens out."""
    s = 2 if spec.dtype == 1 else 4
    B, k, V, G = spec.B, spec.k, spec.V, spec.G
    if mode == "stochastic":
        return B * (2 * k + 1) * V * s + 4 * B * k + 4 * B * k + 4 * B + 4 * B + 4 * B * (k + 1)
    return B * G * (k + 1) * V * s + 4 * B * G * k + 4 * B + 4 * B * (k + 1) + 4 * B


def kernel_name(spec, mode: str) -> str:
    """The kernel that dominates a call: one workgroup per sequence for large
    single-candidate batches, else the row-statistics kernel."""
    if spec.G == 1 and spec.B >= 192:
        return f"k_{mode}_seq"
    return "k_row_stats"


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(workload: int, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    e = tr.get(f"{workload}/{mode}")
    if not e or e.get("kernel_sha") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def to_device(batch, torch, dev):
    import numpy as np
    if batch.spec.dtype == 1:
        t = torch.from_numpy(batch.target.view(np.int16)).to(dev).view(torch.bfloat16)
        d = None if batch.draft is None else \
            torch.from_numpy(batch.draft.view(np.int16)).to(dev).view(torch.bfloat16)
    else:
        t = torch.from_numpy(batch.target).to(dev)
        d = None if batch.draft is None else torch.from_numpy(batch.draft).to(dev)
    return t, d


def time_calls(fn, steps: int, warmup: int, torch):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return start.elapsed_time(end) / steps, wall


def cpu_baseline(batch, mode: str, reps: int = 3):
    """The float64 oracle as it stands, on the host cores, over the whole
    batch (median of `reps`)."""
    from oracle import svo
    s = batch.spec
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        if mode == "stochastic":
            svo.verify_stochastic(batch.target, batch.draft, batch.draft_tokens, batch.u_accept,
                                  batch.u_sample, B=s.B, k=s.k, V=s.V, temperature=s.tau)
        else:
            x = batch.greedy_tokens if batch.greedy_tokens is not None else batch.draft_tokens
            svo.verify_greedy(batch.target, x, B=s.B, G=s.G, k=s.k, V=s.V)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    return {"value": round(s.B / med, 2), "unit": "seqs/s", "cores": svo.num_threads(),
            "kind": "oracle",
            "sample": f"all {s.B} sequences of workload {s.index} ({mode}), median of {reps} "
                      f"runs, {med:.2f} s each"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--mode", choices=["stochastic", "greedy"], default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verification of a batch shards over GPUs "
              "by sequence with no communication, so run one process per GPU on its own "
              "share of sequences.", file=sys.stderr)
        sys.exit(2)

    import torch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ms, _ = time_calls(lambda: dst.copy_(src), args.steps, args.warmup, torch)
        print(json.dumps({"copy_bytes": n, "ms_per_copy": ms,
                          "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))
        return

    from draft_token_verification_10_amd import binding, workloads

    spec = workloads.SPECS[args.workload]
    mode = args.mode or spec.modes[0]
    print(f"# generating workload {spec.index} ({spec.name})", file=sys.stderr, flush=True)
    batch = workloads.make(spec.index)
    t, d = to_device(batch, torch, dev)
    x = torch.from_numpy(batch.draft_tokens).to(dev)
    ua = torch.from_numpy(batch.u_accept).to(dev)
    us = torch.from_numpy(batch.u_sample).to(dev)
    accept = torch.empty(spec.B, dtype=torch.int32, device=dev)
    tokens = torch.empty((spec.B, spec.k + 1), dtype=torch.int32, device=dev)
    best = torch.empty(spec.B, dtype=torch.int32, device=dev)

    if mode == "stochastic":
        # With the p/q diagnostics requested every position of every sequence
        # is evaluated: the full read of all B(2k+1) rows that the headline
        # figure is quoted on, independent of where the first rejection falls.
        dbg = torch.empty((spec.B, spec.k, 2), dtype=torch.float32, device=dev)

        def step():
            binding.sv_verify_stochastic(t, d, x, ua, us, spec.tau, accept_len=accept,
                                         tokens=tokens, dbg_px_qx=dbg)

        def step_early_exit():
            binding.sv_verify_stochastic(t, d, x, ua, us, spec.tau, accept_len=accept,
                                         tokens=tokens)
    else:
        xg = torch.from_numpy(batch.greedy_tokens if batch.greedy_tokens is not None
                              else batch.draft_tokens).to(dev)

        def step():
            binding.sv_verify_greedy(t, xg, accept_len=accept, tokens=tokens, best_cand=best)

    print(f"# timing {args.steps} steps after {args.warmup} warmup", file=sys.stderr, flush=True)
    ms, wall = time_calls(step, args.steps, args.warmup, torch)
    nbytes = algorithmic_bytes(spec, mode)
    gbs = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "verified seqs/sec + achieved HBM GB/s (% of peak), B=256 k=8 V=128256 bf16",
        "value": round(spec.B / (ms * 1e-3), 1),
        "unit": "seqs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if spec.dtype == 1 else "f32",
        "data": "synthetic",
        "config": {"workload": spec.name, "B": spec.B, "k": spec.k, "V": spec.V, "G": spec.G,
                   "mode": mode, "temperature": spec.tau},
        "achieved_GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(spec.index, mode),
                     "algorithmic_bytes": nbytes,
                     "kernel": kernel_name(spec, mode)},
        "wall_s_timed": round(wall, 3),
    }
    if mode == "stochastic" and spec.G == 1 and spec.B >= 192:
        # Separate line: without diagnostics a sequence stops reading at its
        # first rejection.  Bytes are the rows that must then be read (the
        # pairs up to the first rejection, or all rows if none), from the
        # accepted lengths of this batch; the rocprof-counted fetch is in
        # profiles/ when taken.
        ms_x, _ = time_calls(step_early_exit, args.steps, args.warmup, torch)
        a_host = accept.cpu().numpy()
        s_b = 2 if spec.dtype == 1 else 4
        rows = sum(2 * int(a) + 2 if a < spec.k else 2 * spec.k + 1 for a in a_host)
        nb_x = rows * spec.V * s_b + nbytes - spec.B * (2 * spec.k + 1) * spec.V * s_b
        result["early_exit"] = {
            "value": round(spec.B / (ms_x * 1e-3), 1), "unit": "seqs/s",
            "ms_per_step": round(ms_x, 5), "rows_read": rows,
            "bytes_needed": nb_x, "GBps_on_bytes_needed": round(nb_x / (ms_x * 1e-3) / 1e9, 1),
            "mean_accept_len": round(float(a_host.mean()), 4),
            "traffic": traffic_for(spec.index, "stochastic_early_exit")}
    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(batch, mode)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
