"""Calls on several streams at once: the library keeps no state of its own,
so concurrent calls with their own workspaces and outputs must give exactly
what each gives alone (every kernel is deterministic)."""
import numpy as np
import pytest
import torch

from draft_token_verification_10_amd import binding
from draft_token_verification_10_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def bf16(a64):
    bits = W.round_logits(a64, W.BF16)
    return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)


def make_calls(rng):
    """Five different calls (entry points and layouts), each returning a
    function that runs it on a given stream into fresh outputs."""
    calls = []
    # row-split stochastic (B < 192)
    B, k, V = 64, 4, 20000
    t = bf16(rng.standard_normal((B, k + 1, V)) * 3)
    d = bf16(rng.standard_normal((B, k, V)) * 3)
    x = torch.from_numpy(rng.integers(0, V, (B, k)).astype(np.int32)).to(DEV)
    ua = torch.from_numpy(W.exact_uniforms(rng, B * k).reshape(B, k)).to(DEV)
    us = torch.from_numpy(W.exact_uniforms(rng, B)).to(DEV)

    def c0(s, t=t, d=d, x=x, ua=ua, us=us, B=B, k=k, V=V):
        ws = torch.empty(binding.sv_workspace_bytes(B, 1, k, V), dtype=torch.uint8, device=DEV)
        dbg = torch.empty((B, k, 2), dtype=torch.float32, device=DEV)
        a, tok = binding.sv_verify_stochastic(t, d, x, ua, us, 0.9, dbg_px_qx=dbg, workspace=ws,
                                              stream=s)
        return [a, tok, dbg]
    calls.append(c0)
    # one workgroup per sequence (B >= 192), early exit
    B2, k2, V2 = 200, 3, 9000
    t2 = bf16(rng.standard_normal((B2, k2 + 1, V2)) * 2)
    d2 = bf16(rng.standard_normal((B2, k2, V2)) * 2)
    x2 = torch.from_numpy(rng.integers(0, V2, (B2, k2)).astype(np.int32)).to(DEV)
    ua2 = torch.from_numpy(W.exact_uniforms(rng, B2 * k2).reshape(B2, k2)).to(DEV)
    us2 = torch.from_numpy(W.exact_uniforms(rng, B2)).to(DEV)

    def c1(s):
        a, tok = binding.sv_verify_stochastic(t2, d2, x2, ua2, us2, 1.0, stream=s)
        return [a, tok]
    calls.append(c1)
    # greedy, several candidates (row-split)
    B3, G3, k3, V3 = 24, 3, 4, 5000
    t3 = torch.from_numpy(rng.integers(-4, 4, (B3, G3, k3 + 1, V3)).astype(np.float32)).to(DEV)
    x3 = torch.from_numpy(rng.integers(0, V3, (B3, G3, k3)).astype(np.int32)).to(DEV)

    def c2(s):
        ws = torch.empty(binding.sv_workspace_bytes(B3, G3, k3, V3), dtype=torch.uint8,
                         device=DEV)
        return list(binding.sv_verify_greedy(t3, x3, workspace=ws, stream=s))
    calls.append(c2)
    # plain sampling: one pass per row, and sliced rows
    rows = bf16(rng.standard_normal((128, 32000)) * 3)
    rows2 = bf16(rng.standard_normal((16, 200000)) * 3)
    u4 = torch.from_numpy(W.exact_uniforms(rng, 128)).to(DEV)
    u5 = torch.from_numpy(W.exact_uniforms(rng, 16)).to(DEV)

    def c3(s):
        ws = torch.empty(binding.sv_workspace_bytes(16, 1, 0, 200000), dtype=torch.uint8,
                         device=DEV)
        y1 = binding.sv_sample(rows, u4, 1.0, stream=s)
        y2 = binding.sv_sample(rows2, u5, 1.0, workspace=ws, stream=s)
        return [y1, y2]
    calls.append(c3)
    # capped early exit (B >= 192, k >= 6, no diagnostics, a workspace per stream)
    B6, k6, V6 = 256, 8, 4103
    t64 = rng.standard_normal((B6, k6 + 1, V6)) * 3
    t6 = bf16(t64)
    d6 = bf16(t64[:, :k6] + rng.standard_normal((B6, k6, V6)) * 0.05)  # long accepted runs
    x6 = torch.from_numpy(rng.integers(0, V6, (B6, k6)).astype(np.int32)).to(DEV)
    ua6 = torch.from_numpy(W.exact_uniforms(rng, B6 * k6).reshape(B6, k6)).to(DEV)
    us6 = torch.from_numpy(W.exact_uniforms(rng, B6)).to(DEV)

    def c4(s):
        ws = torch.empty(binding.sv_workspace_bytes(B6, 1, k6, V6), dtype=torch.uint8, device=DEV)
        return list(binding.sv_verify_stochastic(t6, d6, x6, ua6, us6, 1.0, workspace=ws, stream=s))
    calls.append(c4)
    return calls


def test_concurrent_streams_match_serial_calls():
    rng = np.random.default_rng(2024)
    calls = make_calls(rng)
    torch.cuda.synchronize()
    cur = torch.cuda.current_stream().cuda_stream
    want = [[o.clone() for o in c(cur)] for c in calls]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in calls]  # default priority
    for rep in range(3):
        print(f"concurrent streams, round {rep}", flush=True)
        got = []
        for c, s in zip(calls, streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                got.append([c(s.cuda_stream) for _ in range(4)])  # several calls deep
        torch.cuda.synchronize()
        for i, (g4, w) in enumerate(zip(got, want)):
            for outs in g4:
                for o, e in zip(outs, w):
                    assert torch.equal(o, e), (rep, i)
