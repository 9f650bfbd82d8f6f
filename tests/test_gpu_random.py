"""Randomised GPU parity: seeded random shapes across the entry points.

The layout a call takes depends on its shape (sequence-resident with 1024 or
512 threads, row-split with spread or one-group finishing, one-pass or
sliced sampling, vector or element-wise loads), with thresholds at 192, 256,
257, 320 and 512 sequences and at several vocabulary sizes.  The fixed cases
of test_gpu_parity.py sit on and around those thresholds; these draw B
(1..700) and V (1..300000) log-uniformly, with random k, dtype, temperature,
padding and alignment, and check every call against the oracle by the same
rules (greedy exact, stochastic within the 1e-5 bands).
"""
import numpy as np
import pytest
import torch

from draft_token_verification_10_amd import binding
from draft_token_verification_10_amd import workloads as W
from oracle import protocol
from test_gpu_parity import (dev, logits_to_device, make_greedy, make_ragged, make_stochastic,
                             run_greedy, run_ragged, run_stochastic)

pytestmark = pytest.mark.gpu

MAX_ELEMS = 6_000_000  # logits per case: keeps every case to about a second of oracle work


def random_cases(n=160, seed=31):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        mode = ["stochastic", "greedy", "ragged", "sample"][(len(cases) // 2) % 4]
        if len(cases) % 2 == 0:  # log-uniform, and uniform over the thresholds
            B = int(np.exp(rng.uniform(0.0, np.log(700.0))))
        else:
            B = int(rng.integers(150, 701))
        V = max(1, int(np.exp(rng.uniform(0.0, np.log(300_000.0)))))
        k = int(rng.integers(1, 9))
        G = int(rng.choice([1, 1, 1, 2, 4])) if mode == "greedy" else 1
        dtype = int(rng.choice([W.F32, W.BF16]))
        tau = float(rng.choice([0.5, 0.8, 1.0, 1.5]))
        pad = int(rng.integers(1, 4)) if rng.random() < 0.25 else 0
        unal = bool(rng.random() < 0.25)
        rows = {"stochastic": B * (2 * k + 1), "greedy": B * G * (k + 1),
                "ragged": B * (2 * k + 1), "sample": B}[mode]
        if rows * (V + pad) > (4 if mode == "sample" else 1) * MAX_ELEMS:
            continue
        cases.append((len(cases), mode, B, G, k, V, dtype, tau, pad, unal))
    return cases


def small_batch_cases(n=40, seed=37):
    """Row-split batches (B < 192) over long rows: the spread draw's group
    count (16 or 8 per sequence), slices cut to its tiles, statistics staged
    or not, sliced sampling with rows dealt to XCDs."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        mode = ["stochastic", "ragged", "sample", "stochastic"][len(cases) % 4]
        B = int(np.exp(rng.uniform(0.0, np.log(191.0))))
        V = int(np.exp(rng.uniform(np.log(2000.0), np.log(300_000.0))))
        k = int(rng.choice([1, 2, 4, 8, 16]))
        dtype = int(rng.choice([W.F32, W.BF16]))
        tau = float(rng.choice([0.7, 1.0]))
        pad = int(rng.integers(1, 9)) if rng.random() < 0.25 else 0
        unal = bool(rng.random() < 0.2)
        rows = B if mode == "sample" else B * (2 * k + 1)
        if rows * (V + pad) > MAX_ELEMS:
            continue
        cases.append((1000 + len(cases), mode, B, 1, k, V, dtype, tau, pad, unal))
    return cases


def wide_long_cases(n=8, seed=41):
    """384 to 512 sequences on rows of at least 160000 bytes: 512-thread
    groups holding the pair streamed last (the early exit, and the full read
    in position order), and ragged batches of uniform length there."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        mode = ["stochastic", "stochastic", "ragged", "stochastic"][len(cases) % 4]
        B = int(rng.integers(384, 513))
        dtype = int(rng.choice([W.F32, W.BF16]))
        s = 2 if dtype == W.BF16 else 4
        V = int(rng.integers(-(-160000 // s), 140_001))
        k = int(rng.integers(1, 4))
        tau = float(rng.choice([0.7, 1.0]))
        pad = int(rng.integers(1, 9)) if rng.random() < 0.25 else 0
        unal = bool(rng.random() < 0.25)
        if B * (2 * k + 1) * (V + pad) > 250_000_000:
            continue
        cases.append((2000 + len(cases), mode, B, 1, k, V, dtype, tau, pad, unal))
    return cases


@pytest.mark.parametrize("case", random_cases() + small_batch_cases() + wide_long_cases(),
                         ids=lambda c: "{}_{}_B{}_G{}_k{}_V{}_{}_t{}_p{}_u{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "bf16" if c[6] else "f32", c[7], c[8], int(c[9])))
def test_random_shape(case):
    i, mode, B, G, k, V, dtype, tau, pad, unal = case
    print(f"random case {case}", flush=True)
    seed = 9000 + i
    if mode == "stochastic":
        t, d, x, ua, us = make_stochastic(seed, B, k, V, dtype, tau)
        rep, _, _ = run_stochastic(t, d, x, ua, us, tau, dtype, pad, unal)
    elif mode == "greedy":
        t, x = make_greedy(seed, B, G, k, V, dtype, ties=bool(i % 3 == 0))
        rep, _ = run_greedy(t, x, dtype, pad, unal)
    elif mode == "ragged":
        cu, t, d, x, ua, us = make_ragged(seed, B, k, V, dtype, tau)
        rep, _ = run_ragged(cu, t, d, x, ua, us, k, tau, dtype, pad, unal)
    else:
        rng = np.random.default_rng(seed)
        rows = W.round_logits(rng.standard_normal((B, V)) * 3, dtype)
        u = W.exact_uniforms(rng, B)
        tt, th, rs = logits_to_device(rows, dtype, pad, unal)
        y = binding.sv_sample(tt, dev(u), tau)
        yg = binding.sv_sample(tt, None, greedy=True)
        torch.cuda.synchronize()
        rep = protocol.compare_sample(th, u, B=B, V=V, temperature=tau, tokens=y.cpu().numpy(),
                                      row_stride=rs)
        repg = protocol.compare_sample(th, None, B=B, V=V, temperature=tau,
                                       tokens=yg.cpu().numpy(), greedy=True, row_stride=rs)
        rep.failures += ["(greedy) " + f for f in repg.failures]
    assert rep.ok(), rep.summary()
