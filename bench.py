"""Benchmark of the verification step on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--mode stochastic]

A step is one sv_* call over one batch of synthetic inputs already resident in
HBM: every row of the hot path (row statistics over all logits, acceptance
ratios, accept-prefix scan, corrective/bonus draw, outputs; plus candidate
selection for the multi-candidate workload).  The default workload is B=256
sequences, k=8 draft tokens, V=128256, bfloat16 logits, stochastic mode.
Prints one JSON line.

Modes:
  stochastic  sv_verify_stochastic (p/q diagnostics on: every row is read);
              an "early_exit" object times the same call without diagnostics
  greedy      sv_verify_greedy
  ragged      sv_verify_stochastic_ragged on the workload with k_b ~ U{1..k}
              draft positions kept per sequence; "early_exit" and "greedy"
              (sv_verify_greedy_ragged) objects beside it
  sample      sv_sample of one token per sequence from target row 0, with a
              "greedy" (argmax) object beside it

Inputs smaller than 512 MB are replicated and the copies rotated from call to
call, so that no call finds its logits in the 256 MB last-level cache (cold
figures); "warm" repeats the timing on one copy.

Other switches, for the profiler:
  --copy-calibration   time a plain device-to-device copy of 1 GiB (the
                       reference kernel for HBM byte counters)
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


def kernel_name(spec, mode: str, diagnostics=True, greedy=False) -> str:
    """The kernel that dominates a call: one workgroup per sequence for large
    single-candidate batches, else the row-statistics kernel."""
    if spec.G == 1 and spec.B >= 192:
        if greedy or mode == "greedy":
            return "k_greedy_seq"
        return "k_stochastic_seq" if diagnostics else "k_stochastic_seq_exit"
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


def n_copies(input_bytes: int, forced) -> int:
    if forced is not None:
        return max(1, forced)
    if input_bytes >= COLD_BYTES:
        return 1
    return min(MAX_COPIES, math.ceil(COLD_BYTES / max(1, input_bytes)))


def cpu_baseline(run, B: int, what: str, reps: int = 3):
    """The float64 oracle as it stands, on the host cores, over the whole
    batch (median of `reps`)."""
    from oracle import svo
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    return {"value": round(B / med, 2), "unit": "seqs/s", "cores": svo.num_threads(),
            "kind": "oracle",
            "sample": f"all {B} sequences of {what}, median of {reps} runs, {med:.2f} s each"}


def line(spec, mode, ms, nbytes, kern, traffic_key, args, wall, extra_config=None):
    gbs = nbytes / (ms * 1e-3) / 1e9
    cfg = {"workload": spec.name, "B": spec.B, "k": spec.k, "V": spec.V, "G": spec.G,
           "mode": mode, "temperature": spec.tau}
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
        "dtype": "bf16" if spec.dtype == 1 else "f32",
        "data": "synthetic",
        "config": cfg,
        "achieved_GBps": round(gbs, 1),
        "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic_for(traffic_key), "algorithmic_bytes": nbytes,
                     "kernel": kern},
        "wall_s_timed": round(wall, 3),
    }


def side(spec, fns, nbytes, kern, traffic_key, args, torch, extra=None):
    ms, _ = time_calls(fns, args.steps, args.warmup, torch)
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"value": round(spec.B / (ms * 1e-3), 1), "unit": "seqs/s",
           "ms_per_step": round(ms, 5), "algorithmic_bytes": nbytes,
           "GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": kern,
           "traffic": traffic_for(traffic_key)}
    out.update(extra or {})
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--mode", choices=["stochastic", "greedy", "ragged", "sample"], default=None)
    ap.add_argument("--copies", type=int, default=None,
                    help="input copies rotated between calls (default: enough to exceed 600 MB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()

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

    spec = workloads.SPECS[args.workload]
    mode = args.mode or spec.modes[0]
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
        kern = kernel_name(spec, "stochastic")
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
        kern = kernel_name(spec, "sample", diagnostics=False)
        traffic_key = f"{spec.index}/sample"
        extra_cfg = {"rows": "target row 0 of every sequence"}
    extra_cfg["input_copies_rotated"] = nc

    print(f"# timing {args.steps} steps after {args.warmup} warmup ({nc} input copies)",
          file=sys.stderr, flush=True)
    ms, wall = time_calls(fns, args.steps, args.warmup, torch)
    result = line(spec, mode, ms, nbytes, kern, traffic_key, args, wall, extra_cfg)
    result["per_call_us"] = per_call_us(fns, min(args.steps, 100), torch)
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
        result["cpu_baseline"] = cpu_baseline(run, B, what)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
