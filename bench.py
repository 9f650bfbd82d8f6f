"""Benchmark of the verification step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--mode stochastic]

A step is one sv_* call over one batch of synthetic inputs already resident in
HBM: every row of the hot path (row statistics over all logits, acceptance
ratios, accept-prefix scan, corrective/bonus draw, outputs; plus candidate
selection for the multi-candidate workload).  The default workload is B=256
sequences, k=8 draft tokens, V=128256, bfloat16 logits, stochastic mode.
Prints one JSON line.  "dtype" is the arithmetic type of the kernels (f32:
bf16 logits are widened on load); the logit type is in "config".

Modes:
  stochastic  sv_verify_stochastic (p/q diagnostics on: every row is read);
              an "early_exit" object times the same call without diagnostics
  greedy      sv_verify_greedy
  ragged      sv_verify_stochastic_ragged on the workload with k_b ~ U{1..k}
              draft positions kept per sequence; "early_exit" and "greedy"
              (sv_verify_greedy_ragged) objects beside it
  sample      sv_sample of one token per sequence from target row 0, with a
              "greedy" (argmax) object beside it
  tree        sv_verify_greedy_tree on B=32 sequences of a fixed 64-node
              EAGLE-style draft tree (V=128256, bf16)
  commit      sv_commit of the workload's verified step (B sequences, k+1
              token slots): a launch-bound kernel, timed on its own

Where rocprofv3 counts for the current kernel source are committed, each
line and side object also gives "fetched_GBps": the rate on the bytes the
counters saw moving (for early exit, the denominator that matches what it
reads).  Every HBM-bound line also carries "achievable_read": the rate of a plain
read with the same loads (sv_stream_read over 2 GiB) and the path's fraction
of it, beside the fraction of the 8 TB/s peak.

Order: inputs are generated and placed in HBM, the achievable read rate is
measured (about 0.2 s of streaming), then W warm-up calls and the K timed
calls run back to back between two events.  Measuring the read rate first
also takes the GPU past the dip its clock shows in the first ~20 ms of load
after idle (per-XCD clock about 2.3 -> 2.06 -> 2.45 GHz), which would
otherwise fall on the timed calls of the exponential-heavy stochastic kernels.

Inputs smaller than 512 MB are replicated and the copies rotated from call to
call, so that no call finds its logits in the 256 MB last-level cache (cold
figures); "warm" repeats the timing on one copy.

Other switches, for the profiler:
  --copy-calibration   time a plain device-to-device copy of 1 GiB (the
                       reference kernel for HBM byte counters)
  --record-traffic KEY --fetch-csv F --write-csv W --kernels 'K1;K2' [--source S]
                       (no GPU) store one call's HBM bytes from a FETCH_SIZE
                       and a WRITE_SIZE rocprofv3 run in profiles/traffic.json
  --no-cpu-baseline    skip the CPU oracle timing
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
KERNEL_SRC = os.path.join(ROOT, "draft_token_verification_10_amd", "csrc", "sv_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
COLD_BYTES = 600_000_000  # rotate copies until the inputs exceed this
MAX_COPIES = 600


def elem_size(spec) -> int:
    return 2 if spec.dtype == 1 else 4


def algorithmic_bytes(spec, mode: str, kb=None, greedy=False) -> int:
    """Bytes the method itself must move per call: every logit row once, the
    draft tokens and uniforms in, accept_len and tokens out."""
    s = elem_size(spec)
    B, k, V, G = spec.B, spec.k, spec.V, spec.G
    if mode == "stochastic":
        return B * (2 * k + 1) * V * s + 4 * B * k + 4 * B * k + 4 * B + 4 * B + 4 * B * (k + 1)
    if mode == "greedy":
        return B * G * (k + 1) * V * s + 4 * B * G * k + 4 * B + 4 * B * (k + 1) + 4 * B
    if mode == "ragged":
        n = int(sum(kb))
        io = 4 * (B + 1) + 4 * B + 4 * B * (k + 1)  # cu, accept_len, tokens out
        if greedy:
            return (n + B) * V * s + 4 * n + io
        return (2 * n + B) * V * s + 4 * n + 4 * n + 4 * B + io
    if mode == "sample":
        return B * V * s + (0 if greedy else 4 * B) + 4 * B
    raise ValueError(mode)


def tree_bytes(B: int, N: int, V: int, s: int) -> int:
    """Every node row once, node tokens and parents in, accept_len, tokens and
    path out."""
    return B * N * V * s + 8 * B * N + 4 * B + 8 * B * N


def commit_bytes(accept, W: int) -> int:
    """accept_len, the token rows and seq_len read; the appended tokens,
    seq_len and the next token written."""
    B = len(accept)
    return 4 * B + 4 * B * W + 4 * B + 4 * int(sum(int(a) + 1 for a in accept)) + 4 * B + 4 * B


def sample_one_pass(B: int, V: int, elem_bytes: int) -> bool:
    """The library's layout choice for sv_sample with u on contiguous rows:
    one workgroup per row (1024 threads up to 256 rows, 512 beyond) where
    that is faster, else sliced rows."""
    chunks = V // (16 // elem_bytes)
    if B > 256:
        return (B <= 512 and (chunks + 511) // 512 <= 32 and
                (V <= 40960 or (B >= 320 and V <= 98304)))
    return (chunks + 1023) // 1024 <= 32 and V <= 40960 + 352 * B


def kernel_name(spec, mode: str, diagnostics=True, greedy=False, uniform=True) -> str:
    """The kernel that dominates a call, following the library's layout
    choice: one workgroup per sequence for large single-candidate batches
    (not for ragged batches of unequal lengths read in full), one per row for
    plain sampling where that is faster, else the row-statistics kernel."""
    if mode == "sample" and not greedy:
        from draft_token_verification_10_amd.workloads import BF16
        es = 2 if spec.dtype == BF16 else 4
        return "k_sample_seq" if sample_one_pass(spec.B, spec.V, es) else "k_row_stats"
    if spec.G == 1 and spec.B >= 192:
        if greedy or mode == "greedy":
            return "k_greedy_seq"
        if not diagnostics:
            if spec.k >= 6 and spec.B <= 1024:  # capped pass, then the spread continuation
                return "k_stochastic_seq_exit (capped) + k_exit_stats + k_draw_tiles"
            return "k_stochastic_seq_exit"
        if not uniform:
            return "k_row_stats"
        # the full read runs in position order in the early-exit kernel's
        # full-read variant up to 256 sequences (one 1024-thread group each),
        # and from 384 to 512 sequences with rows of at least 160000 bytes
        # (512-thread groups, two per CU)
        from draft_token_verification_10_amd.workloads import BF16
        row_bytes = spec.V * (2 if spec.dtype == BF16 else 4)
        if spec.B <= 256 or (384 <= spec.B <= 512 and row_bytes >= 160000):
            return "k_stochastic_seq_exit (full read)"
        return "k_stochastic_seq"
    return "k_row_stats"


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_for(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they are missing or were taken on a different kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        return None
    e = tr.get(key)
    if not e or e.get("kernel_sha") != kernel_hash():
        return None
    return e.get("bytes_per_launch")


def counter_kib(csv_path: str, kernel: str) -> float:
    """Median over dispatches of the counter in a rocprofv3 counter-collection
    CSV (one counter per run), for the kernels whose name contains `kernel`."""
    import csv
    import statistics
    vals = []
    with open(csv_path, newline="") as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatch of {kernel!r} in {csv_path}")
    return statistics.median(vals)


def record_traffic(key: str, fetch_csv: str, write_csv: str, kernels: list, source: str) -> dict:
    """Store the HBM bytes one call moves, from a FETCH_SIZE run and a
    WRITE_SIZE run of rocprofv3 (KiB per dispatch, summed over the call's
    kernels), in profiles/traffic.json under `key` with the kernel source
    hash.  Key "_calibration" takes a plain 1 GiB device copy
    (bench.py --copy-calibration) and stores the factor that turns each
    counter into bytes; the other keys are scaled by it."""
    try:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
    except (OSError, ValueError):
        tr = {}
    fk = sum(counter_kib(fetch_csv, k) for k in kernels)
    wk = sum(counter_kib(write_csv, k) for k in kernels)
    if key == "_calibration":
        n = 1 << 30
        entry = {"kernel": " + ".join(kernels), "copy_bytes": n,
                 "fetch_kib": fk, "write_kib": wk,
                 "fetch_scale": round(n / (fk * 1024), 5), "write_scale": round(n / (wk * 1024), 5),
                 "source": source}
    else:
        cal = tr.get("_calibration")
        if not cal:
            raise SystemExit("record the copy calibration (key _calibration) first")
        fb = int(round(fk * 1024 * cal["fetch_scale"]))
        wb = int(round(wk * 1024 * cal["write_scale"]))
        entry = {"kernel": " + ".join(kernels), "kernel_sha": kernel_hash(),
                 "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
                 "bytes_per_launch": fb + wb, "fetch_scale": cal["fetch_scale"],
                 "write_scale": cal["write_scale"], "source": source}
        if len(kernels) > 1:
            entry["per"] = "call (all kernels of the call)"
    tr[key] = entry
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(tr, f, indent=1)
        f.write("\n")
    return entry


def logits_to_device(a, dtype, torch, dev):
    import numpy as np
    if a is None:
        return None
    if dtype == 1:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def time_calls(fns, steps: int, warmup: int, torch):
    """Mean time per call of `steps` back-to-back calls (cycling through
    `fns`), between two events on the current stream."""
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(steps):
        fns[i % len(fns)]()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return start.elapsed_time(end) / steps, wall


def per_call_us(fns, steps: int, torch):
    """Each call between its own pair of events: p10 / median / p90 in µs."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        fns[i % len(fns)]()
        b.record(stream)
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) * 1e3 for a, b in ev)

    def q(f):
        return round(t[min(len(t) - 1, int(f * len(t)))], 2)
    return {"p10": q(0.1), "median": q(0.5), "p90": q(0.9)}


def graph_us(fns, calls: int, replays: int, torch):
    """Device time per call without host launch overhead: `calls` calls
    (cycling through `fns`) captured once in a HIP graph on a side stream of
    default priority, replayed `replays` times between two events."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(3):  # workspaces are allocated here, outside the capture
            fns[i % len(fns)]()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(calls):
            fns[i % len(fns)]()
    g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(replays):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) * 1e3 / (calls * replays)


def n_copies(input_bytes: int, forced) -> int:
    if forced is not None:
        return max(1, forced)
    if input_bytes >= COLD_BYTES:
        return 1
    return min(MAX_COPIES, math.ceil(COLD_BYTES / max(1, input_bytes)))


def cpu_baseline(run, B: int, what: str, nbytes: int, gpu_value: float, min_reps: int = 3,
                 target_s: float = 10.0, max_s: float = 30.0):
    """The float64 oracle as it stands, on the host cores: whole-batch passes
    repeated until about `target_s` seconds of work (at least `min_reps`
    passes, never starting one past `max_s`); the median pass is reported,
    with the oracle's rate on the same algorithmic bytes as the GPU figure
    and the GPU/CPU ratio."""
    from oracle import svo
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
        spent = time.perf_counter() - t_start
        if len(times) >= min_reps and (spent >= target_s or spent + times[-1] > max_s):
            break
    times.sort()
    med = times[len(times) // 2]
    value = B / med
    out = {"value": round(value, 2), "unit": "seqs/s", "cores": svo.num_threads(),
           "kind": "oracle",
           "sample": f"all {B} sequences of {what} per pass, {len(times)} passes "
                     f"({sum(times):.1f} s), median pass {med:.3f} s",
           "GBps": round(nbytes / med / 1e9, 3),
           "gpu_speedup": round(gpu_value / value, 1),
           "threads": svo.num_threads(), **host_cpu()}
    # the same oracle on one thread: one whole-batch pass
    threads = svo.num_threads()
    svo.set_num_threads(1)
    try:
        est = med * threads
        t0 = time.perf_counter()
        run()
        one = time.perf_counter() - t0
    finally:
        svo.set_num_threads(threads)
    out["single_thread"] = {"value": round(B / one, 2), "unit": "seqs/s", "cores": 1,
                            "GBps": round(nbytes / one / 1e9, 3),
                            "gpu_speedup": round(gpu_value / (B / one), 1),
                            "sample": f"one pass over all {B} sequences ({one:.1f} s; "
                                      f"{est:.1f} s expected from the threaded median)"}
    return out


def achievable_read(torch, binding, dev, nbytes: int = 2 << 30, steps: int = 20) -> dict:
    """The read rate a plain stream with the logit kernels' own loads sustains
    (sv_stream_read: every byte of a 2 GiB buffer, eight times the last-level
    cache, read once by N workgroups each taking one contiguous share), for
    several N; the best is the practical ceiling reported beside the peak.
    Run before the timed steps: its ~0.2 s of streaming also carries the GPU
    past the clock dip of its first ~20 ms of load after idle, which the
    exponential-heavy stochastic kernels would otherwise be timed in."""
    buf = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
    out = torch.zeros(4096, dtype=torch.int32, device=dev)
    sweep = {}
    for blocks in (256, 512, 1024, 2048, 4096):
        ms, _ = time_calls([lambda b=blocks: binding.sv_stream_read(buf, b, out)], steps, 3,
                           torch)
        sweep[str(blocks)] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    best = max(sweep, key=sweep.get)
    del buf
    return {"GBps": sweep[best], "frac_of_peak": round(sweep[best] / HBM_PEAK_GBS, 4),
            "workgroups": int(best), "bytes": nbytes, "kernel": "k_stream_read",
            "GBps_by_workgroups": sweep}


def with_path_frac(ach: dict, achieved_gbs: float) -> dict:
    out = dict(ach)
    out["path_frac_of_achievable"] = round(achieved_gbs / ach["GBps"], 4)
    return out


def host_cpu() -> dict:
    """The measuring host: CPU model, logical CPUs, physical cores (distinct
    (package, core) pairs in /proc/cpuinfo) and the CPUs this process may
    run on."""
    model, cores = None, set()
    phys = core = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                key, _, val = ln.partition(":")
                key, val = key.strip(), val.strip()
                if key == "model name" and model is None:
                    model = val
                elif key == "physical id":
                    phys = val
                elif key == "core id":
                    core = val
                elif not key and phys is not None and core is not None:
                    cores.add((phys, core))
                    phys = core = None
    except OSError:
        pass
    if phys is not None and core is not None:
        cores.add((phys, core))
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "physical_cores": len(cores) or None, "cpus_allowed": allowed}


def line(spec, mode, ms, nbytes, kern, traffic_key, args, wall, extra_config=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    cfg = {"workload": spec.name, "B": spec.B, "k": spec.k, "V": spec.V, "G": spec.G,
           "logits": "bf16" if spec.dtype == 1 else "f32", "mode": mode,
           "temperature": spec.tau}
    cfg.update(extra_config or {})
    return {
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
        "dtype": "f32",
        "data": "synthetic",
        "config": cfg,
        "achieved_GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(traffic_key), "algorithmic_bytes": nbytes,
                     "kernel": kern},
        "wall_s_timed": round(wall, 3),
        **fetched_rate(traffic_for(traffic_key), ms),
    }


def fetched_rate(traffic, ms):
    """GB/s and fraction of the peak on the bytes rocprofv3 counted moving
    (null without counts for the current kernel source)."""
    if traffic is None:
        return {"fetched_GBps": None, "fetched_frac": None}
    gbs = traffic / (ms * 1e-3) / 1e9
    return {"fetched_GBps": round(gbs, 1), "fetched_frac": round(gbs / HBM_PEAK_GBS, 4)}


def side(spec, fns, nbytes, kern, traffic_key, args, torch, extra=None):
    ms, _ = time_calls(fns, args.steps, args.warmup, torch)
    gbs = nbytes / (ms * 1e-3) / 1e9
    traffic = traffic_for(traffic_key)
    out = {"value": round(spec.B / (ms * 1e-3), 1), "unit": "seqs/s",
           "ms_per_step": round(ms, 5), "algorithmic_bytes": nbytes,
           "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": kern,
           "traffic": traffic}
    out.update(fetched_rate(traffic, ms))
    out.update(extra or {})
    return out


def bench_tree(args, torch, dev, binding, workloads):
    import numpy as np
    print("# generating the draft-tree batch", file=sys.stderr, flush=True)
    tb = workloads.tree_batch()
    B, N, V = tb.target.shape
    s_b = 2 if tb.dtype == 1 else 4
    nc = n_copies(tb.target.nbytes, args.copies)
    t0 = logits_to_device(tb.target, tb.dtype, torch, dev)
    ts = [t0] + [t0.clone() for _ in range(nc - 1)]
    x = torch.from_numpy(tb.node_tokens).to(dev)
    par = torch.from_numpy(tb.parents).to(dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    fns = [(lambda t=t: binding.sv_verify_greedy_tree(t, x, par, accept_len=acc, tokens=tok,
                                                      path=path)) for t in ts]
    ach = achievable_read(torch, binding, dev)
    ms, wall = time_calls(fns, args.steps, args.warmup, torch)
    nbytes = tree_bytes(B, N, V, s_b)
    gbs = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "verified seqs/sec + achieved HBM GB/s (% of peak), greedy draft tree",
        "value": round(B / (ms * 1e-3), 1), "unit": "seqs/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"tree_B{B}_N{N}_V{V}_bf16", "B": B, "N": N, "V": V,
                   "logits": "bf16" if tb.dtype == 1 else "f32",
                   "tree_levels": list(workloads.TREE_LEVELS), "mode": "tree",
                   "input_copies_rotated": nc},
        "achieved_GBps": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for("tree"), "algorithmic_bytes": nbytes,
                     "kernel": "k_row_stats"},
        "wall_s_timed": round(wall, 3),
        **fetched_rate(traffic_for("tree"), ms),
        "per_call_us": per_call_us(fns, min(args.steps, 100), torch),
        "mean_accepted_depth": round(float(acc.float().mean().item()), 4),
    }
    result["achievable_read"] = with_path_frac(ach, gbs)
    if not args.no_cpu_baseline:
        from oracle import svo
        result["cpu_baseline"] = cpu_baseline(
            lambda: svo.verify_greedy_tree(tb.target, tb.node_tokens, tb.parents, B=B, N=N, V=V),
            B, f"the draft-tree batch (B={B}, N={N})", nbytes, result["value"])
    print(json.dumps(result), flush=True)


def bench_commit(args, torch, dev, binding, workloads, spec):
    """The commit of workload `spec`'s greedy verification outputs."""
    import numpy as np
    print(f"# generating workload {spec.index} for its verified step", file=sys.stderr, flush=True)
    batch = workloads.make(spec.index)
    B, k = spec.B, spec.k
    t = logits_to_device(batch.target, spec.dtype, torch, dev)
    x = torch.from_numpy(batch.draft_tokens).to(dev)
    acc, tok = binding.sv_verify_greedy(t, x)[:2]
    cap = 16384  # room for every commit of the run: none is cut short by the capacity
    hist = torch.zeros((B, cap), dtype=torch.int32, device=dev)
    seq_len = torch.zeros(B, dtype=torch.int32, device=dev)
    ids = torch.zeros((B, k + 1), dtype=torch.int32, device=dev)

    def step():
        binding.sv_commit(acc, tok, seq_len, hist, ids[:, 0])

    a_host = acc.cpu().numpy()
    nbytes = commit_bytes(a_host, k + 1)
    # Device time: 50 commits captured in a graph, replayed 20 times.
    calls, replays = 50, 20
    seq_len.zero_()
    us_graph = graph_us([step], calls, replays, torch)
    seq_len.zero_()
    ms, wall = time_calls([step], min(args.steps, (cap - 1) // (k + 1) - args.warmup),
                          args.warmup, torch)
    result = {
        "metric": "commit of a verified step: µs per call on the device (graph replay)",
        "value": round(us_graph, 3), "unit": "us", "n_gpus": 1,
        "steps": calls, "warmup": 3, "ms_per_step": round(us_graph * 1e-3, 6),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int32", "data": "synthetic",
        "config": {"workload": spec.name, "B": B, "W": k + 1, "mode": "commit"},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (us_graph * 1e-6) / 1e9, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (us_graph * 1e-6) / 1e9 / HBM_PEAK_GBS, 6),
                     "traffic": None, "algorithmic_bytes": nbytes, "kernel": "k_commit"},
        "eager_us_per_call": round(ms * 1e3, 3),
        "note": "a launch-bound kernel: the eager figure is the Python binding's call rate",
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--mode", choices=["stochastic", "greedy", "ragged", "sample", "tree",
                                       "commit"], default=None)
    ap.add_argument("--copies", type=int, default=None,
                    help="input copies rotated between calls (default: enough to exceed 600 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--record-traffic", metavar="KEY", default=None,
                    help="store a call's HBM bytes from two rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--fetch-csv", default=None)
    ap.add_argument("--write-csv", default=None)
    ap.add_argument("--kernels", default=None,
                    help="kernel names of one call, as in the CSVs, separated by ';' "
                         "(template arguments hold commas)")
    ap.add_argument("--source", default="", help="the profile summary quoting the counts")
    args = ap.parse_args()

    if args.record_traffic:
        if not (args.fetch_csv and args.write_csv and args.kernels):
            ap.error("--record-traffic needs --fetch-csv, --write-csv and --kernels")
        e = record_traffic(args.record_traffic, args.fetch_csv, args.write_csv,
                           args.kernels.split(";"), args.source)
        print(json.dumps({args.record_traffic: e}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the verification of a batch shards over GPUs "
              "by sequence with no communication, so run one process per GPU on its own "
              "share of sequences.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        ms, _ = time_calls([lambda: dst.copy_(src)], args.steps, args.warmup, torch)
        print(json.dumps({"copy_bytes": n, "ms_per_copy": ms,
                          "GBps_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}))
        return

    from draft_token_verification_10_amd import binding, workloads

    if args.mode == "tree":
        return bench_tree(args, torch, dev, binding, workloads)
    spec = workloads.SPECS[args.workload]
    mode = args.mode or spec.modes[0]
    if mode == "commit":
        return bench_commit(args, torch, dev, binding, workloads, spec)
    if mode in ("ragged",) and (spec.G != 1 or spec.index == 4):
        sys.exit("ragged mode needs a single-candidate stochastic workload")
    print(f"# generating workload {spec.index} ({spec.name}), mode {mode}", file=sys.stderr,
          flush=True)
    batch = workloads.make(spec.index)
    B = spec.B
    s_b = elem_size(spec)

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    accept = torch.empty(B, dtype=torch.int32, device=dev)
    tokens = torch.empty((B, spec.k + 1), dtype=torch.int32, device=dev)
    best = torch.empty(B, dtype=torch.int32, device=dev)
    extra_cfg = {}
    sides = {}

    if mode in ("stochastic", "greedy"):
        t_h, d_h = batch.target, batch.draft
        in_bytes = t_h.nbytes + (0 if d_h is None or mode == "greedy" else d_h.nbytes)
        nc = n_copies(in_bytes, args.copies)
        t0 = logits_to_device(t_h, spec.dtype, torch, dev)
        ts = [t0] + [t0.clone() for _ in range(nc - 1)]
        x = up(batch.draft_tokens)
        if mode == "stochastic":
            d0 = logits_to_device(d_h, spec.dtype, torch, dev)
            ds = [d0] + [d0.clone() for _ in range(nc - 1)]
            ua, us = up(batch.u_accept), up(batch.u_sample)
            # With the p/q diagnostics requested every position of every
            # sequence is evaluated: the full read of all B(2k+1) rows that the
            # headline figure is quoted on, whatever the first rejection.
            dbg = torch.empty((B, spec.k, 2), dtype=torch.float32, device=dev)
            fns = [(lambda t=t, d=d: binding.sv_verify_stochastic(
                t, d, x, ua, us, spec.tau, accept_len=accept, tokens=tokens, dbg_px_qx=dbg))
                for t, d in zip(ts, ds)]
            fns_x = [(lambda t=t, d=d: binding.sv_verify_stochastic(
                t, d, x, ua, us, spec.tau, accept_len=accept, tokens=tokens))
                for t, d in zip(ts, ds)]
            nbytes = algorithmic_bytes(spec, "stochastic")
            kern = kernel_name(spec, "stochastic")
        else:
            xg = up(batch.greedy_tokens if batch.greedy_tokens is not None
                    else batch.draft_tokens)
            fns = [(lambda t=t: binding.sv_verify_greedy(t, xg, accept_len=accept, tokens=tokens,
                                                         best_cand=best)) for t in ts]
            nbytes = algorithmic_bytes(spec, "greedy")
            kern = kernel_name(spec, "greedy")
        traffic_key = f"{spec.index}/{mode}"
    elif mode == "ragged":
        rb = workloads.ragged(batch)
        in_bytes = rb.target.nbytes + rb.draft.nbytes
        nc = n_copies(in_bytes, args.copies)
        t0 = logits_to_device(rb.target, spec.dtype, torch, dev)
        d0 = logits_to_device(rb.draft, spec.dtype, torch, dev)
        ts = [t0] + [t0.clone() for _ in range(nc - 1)]
        ds = [d0] + [d0.clone() for _ in range(nc - 1)]
        x, cu, ua, us = up(rb.draft_tokens), up(rb.cu), up(rb.u_accept), up(rb.u_sample)
        dbg = torch.empty((int(rb.cu[-1]), 2), dtype=torch.float32, device=dev)
        k = spec.k
        fns = [(lambda t=t, d=d: binding.sv_verify_stochastic_ragged(
            t, d, x, cu, ua, us, k, spec.tau, accept_len=accept, tokens=tokens, dbg_px_qx=dbg))
            for t, d in zip(ts, ds)]
        fns_x = [(lambda t=t, d=d: binding.sv_verify_stochastic_ragged(
            t, d, x, cu, ua, us, k, spec.tau, accept_len=accept, tokens=tokens))
            for t, d in zip(ts, ds)]
        fns_g = [(lambda t=t: binding.sv_verify_greedy_ragged(t, x, cu, k, accept_len=accept,
                                                              tokens=tokens)) for t in ts]
        nbytes = algorithmic_bytes(spec, "ragged", rb.kb)
        kern = kernel_name(spec, "ragged", uniform=bool((rb.kb == spec.k).all()))
        traffic_key = f"{spec.index}/ragged"
        extra_cfg = {"draft_len": "k_b ~ U{1..k}", "total_draft": int(rb.cu[-1]),
                     "mean_k_b": round(float(rb.kb.mean()), 4)}
    else:  # sample
        rows, u = workloads.sample_rows(batch)
        nc = n_copies(rows.nbytes, args.copies)
        t0 = logits_to_device(rows, spec.dtype, torch, dev)
        ts = [t0] + [t0.clone() for _ in range(nc - 1)]
        ud = up(u)
        ytok = torch.empty(B, dtype=torch.int32, device=dev)
        fns = [(lambda t=t: binding.sv_sample(t, ud, spec.tau, tokens=ytok)) for t in ts]
        fns_g = [(lambda t=t: binding.sv_sample(t, None, greedy=True, tokens=ytok)) for t in ts]
        nbytes = algorithmic_bytes(spec, "sample")
        kern = kernel_name(spec, "sample")
        traffic_key = f"{spec.index}/sample"
        extra_cfg = {"rows": "target row 0 of every sequence"}
    extra_cfg["input_copies_rotated"] = nc

    print("# achievable read rate (sv_stream_read over 2 GiB)", file=sys.stderr, flush=True)
    ach = achievable_read(torch, binding, dev)
    print(f"# timing {args.steps} steps after {args.warmup} warmup ({nc} input copies)",
          file=sys.stderr, flush=True)
    ms, wall = time_calls(fns, args.steps, args.warmup, torch)
    result = line(spec, mode, ms, nbytes, kern, traffic_key, args, wall, extra_cfg)
    result["per_call_us"] = per_call_us(fns, min(args.steps, 100), torch)
    # the device time of a call without the binding's host overhead (20
    # calls captured in a graph, 10 replays), beside the eager mean
    result["graph_us_per_call"] = round(graph_us(fns, 20, 10, torch), 2)
    if nc > 1:
        ms_w, _ = time_calls(fns[:1], args.steps, args.warmup, torch)
        result["warm"] = {"ms_per_step": round(ms_w, 5),
                          "value": round(B / (ms_w * 1e-3), 1),
                          "GBps": round(nbytes / (ms_w * 1e-3) / 1e9, 1)}

    if mode in ("stochastic", "ragged") and spec.G == 1 and B >= 192:
        # Without diagnostics a sequence stops reading at its first rejection.
        # Bytes are the rows that must then be read (the pairs up to the first
        # rejection, or all rows if none), from the accepted lengths of this
        # batch.
        a_host = accept.cpu().numpy()
        kb = rb.kb if mode == "ragged" else np.full(B, spec.k)
        rows_needed = sum(2 * int(a) + 2 if a < int(kk) else 2 * int(kk) + 1
                          for a, kk in zip(a_host, kb))
        full_rows = int(sum(2 * kb + 1))
        nb_x = nbytes - (full_rows - rows_needed) * spec.V * s_b
        sides["early_exit"] = side(
            spec, fns_x, nb_x, kernel_name(spec, mode, diagnostics=False),
            f"{traffic_key}_early_exit", args, torch,
            {"rows_read": rows_needed, "mean_accept_len": round(float(a_host.mean()), 4),
             "note": "algorithmic_bytes counts only the rows a first-rejection exit must read"})
    if mode in ("ragged", "sample"):
        gb = algorithmic_bytes(spec, mode, rb.kb if mode == "ragged" else None, greedy=True)
        sides["greedy"] = side(spec, fns_g, gb, kernel_name(spec, mode, greedy=True),
                               f"{traffic_key}_greedy", args, torch)
    result.update(sides)
    result["achievable_read"] = with_path_frac(ach, result["achieved_GBps"])

    if not args.no_cpu_baseline:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        from oracle import svo
        what = f"workload {spec.index} ({mode})"
        if mode == "stochastic":
            run = lambda: svo.verify_stochastic(batch.target, batch.draft, batch.draft_tokens,  # noqa
                                                batch.u_accept, batch.u_sample, B=B, k=spec.k,
                                                V=spec.V, temperature=spec.tau)
        elif mode == "greedy":
            xg_h = batch.greedy_tokens if batch.greedy_tokens is not None else batch.draft_tokens
            run = lambda: svo.verify_greedy(batch.target, xg_h, B=B, G=spec.G, k=spec.k,  # noqa
                                            V=spec.V)
        elif mode == "ragged":
            run = lambda: svo.verify_stochastic_ragged(rb.target, rb.draft, rb.draft_tokens,  # noqa
                                                       rb.cu, rb.u_accept, rb.u_sample,
                                                       k_max=spec.k, V=spec.V,
                                                       temperature=spec.tau)
        else:
            run = lambda: svo.sample(rows, u, B=B, V=spec.V, temperature=spec.tau)  # noqa
        result["cpu_baseline"] = cpu_baseline(run, B, what, nbytes, result["value"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
