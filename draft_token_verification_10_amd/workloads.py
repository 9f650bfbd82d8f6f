"""Seeded synthetic inputs for the verification step.

This module only draws random inputs; it contains none of the verification
arithmetic.  Both the GPU library's tests/benchmark and the CPU oracle are fed
from here.

Five workloads, each with its own seed ``10_000 + index`` and six independent
streams (target logits, draft noise, spikes/candidates, draft-token noise,
acceptance uniforms, sample uniforms).  Every sequence ``b`` draws from its own
child of each stream (``SeedSequence(10_000 + index, spawn_key=(stream, b))``),
so any subset of sequences can be regenerated on its own and the batch can be
built in parallel.

Logits are drawn in float64, then rounded to float32 (round to nearest even)
and, for bf16 workloads, to bfloat16 (round to nearest even on the float32 bit
pattern).  Draft tokens are sampled from softmax(rounded draft logits / tau)
with the Gumbel-max construction (argmax of logits/tau plus independent Gumbel
noise), which draws exactly from that softmax.  Uniforms are exact float32
values ``m * 2**-24`` with ``m`` uniform on ``[0, 2**24)``, so they lie in
``[0, 1)``.

Two derived inputs reuse a workload's rows: a ragged batch (``ragged``), in
which sequence b keeps only its first k_b ~ U{1..k} draft positions (drawn
from a seventh stream), packed without gaps; and a sampling batch
(``sample_rows``), the first target row of every sequence with its sample
uniform.  A draft-tree batch (``tree_batch``) holds a fixed 64-node
EAGLE-style tree per sequence.

The workloads:

0. ``B=1, k=4, V=32000`` fp32, tau 1: target ~ N(0, 3^2) i.i.d., draft =
   target + N(0, 0.5^2); stochastic and greedy.
1. ``B=64, k=4, V=128256`` bf16, tau 1: target ~ N(0, 3^2), draft = target +
   N(0, 1); stochastic.
2. ``B=256, k=8, V=128256`` bf16, tau 1: target ~ N(0, 4^2) with exactly
   floor(0.01 V) distinct entries per target row raised by 10 (peaked rows);
   draft = target + N(0, 1.5^2); stochastic, and greedy on a second token set
   (the draft's own argmax, which gives long accepted prefixes).
3. ``B=512, k=3, V=129280`` bf16, tau 0.7 on both sides: target ~ N(0, 3^2);
   per-sequence draft noise sigma_b ~ U[0.2, 3.0] (a spread of acceptance
   rates); stochastic.
4. ``B=32, G=16, n=4, V=32000`` fp32 multi-candidate greedy (Lookahead-style
   n-gram verification): target ~ N(0, 3^2) for every candidate position;
   candidate tokens uniform over V, except that 4 of the 16 candidates of each
   sequence (a seeded choice) have their first j ~ U{1..4} tokens replaced by
   the argmax of the matching target rows.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

F32 = 0
BF16 = 1

# stream indices (S_LEN: per-sequence draft lengths of the ragged variant)
S_TARGET, S_DRAFT, S_SPIKE, S_TOKEN, S_UACC, S_USAMP, S_LEN = range(7)


@dataclass(frozen=True)
class Spec:
    index: int
    name: str
    B: int
    k: int
    V: int
    dtype: int
    tau: float
    G: int = 1
    modes: tuple = ("stochastic",)


SPECS = [
    Spec(0, "B1_k4_V32000_f32", 1, 4, 32000, F32, 1.0, modes=("stochastic", "greedy")),
    Spec(1, "B64_k4_V128256_bf16", 64, 4, 128256, BF16, 1.0),
    Spec(2, "B256_k8_V128256_bf16_peaked", 256, 8, 128256, BF16, 1.0,
         modes=("stochastic", "greedy")),
    Spec(3, "B512_k3_V129280_bf16_tau0.7", 512, 3, 129280, BF16, 0.7),
    Spec(4, "B32_G16_n4_V32000_f32_lookahead", 32, 4, 32000, F32, 1.0, G=16,
         modes=("greedy",)),
]


@dataclass
class Batch:
    """A batch of verification inputs (host numpy arrays).

    target: [B][k+1][V] (greedy multi-candidate: [B][G][k+1][V]); float32, or
    uint16 holding bfloat16 bit patterns.  draft: [B][k][V] or None.
    draft_tokens: int32 [B][k] ([B][G][k]).  u_accept: float32 [B][k];
    u_sample: float32 [B].  greedy_tokens: optional second token set for greedy
    mode ([B][k]).
    """
    spec: Spec
    target: np.ndarray
    draft: np.ndarray | None
    draft_tokens: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray
    greedy_tokens: np.ndarray | None = None
    seqs: np.ndarray = field(default=None)


def rng_for(index: int, stream: int, b: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(10_000 + index, spawn_key=(stream, b)))


def to_f32(x64: np.ndarray) -> np.ndarray:
    return x64.astype(np.float32)


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Inputs are finite or infinite (no NaN)."""
    bits = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (bits >> 16) & np.uint32(1)
    return ((bits + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)


def bf16_bits_to_f64(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_logits(x64: np.ndarray, dtype: int) -> np.ndarray:
    x32 = to_f32(x64)
    return f32_to_bf16_bits(x32) if dtype == BF16 else x32


def as_f64(stored: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_bits_to_f64(stored) if dtype == BF16 else stored.astype(np.float64)


def exact_uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    m = rng.integers(0, 1 << 24, size=n, dtype=np.int64)
    return (m.astype(np.float64) * 2.0 ** -24).astype(np.float32)


def gumbel_max(rng: np.random.Generator, logits64: np.ndarray, tau: float) -> np.ndarray:
    """One draw per row from softmax(logits/tau) (Gumbel-max)."""
    u = rng.random(logits64.shape)
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    return np.argmax(logits64 / tau + g, axis=-1).astype(np.int32)


def _sequence(spec: Spec, b: int):
    idx, k, V = spec.index, spec.k, spec.V
    rt = rng_for(idx, S_TARGET, b)
    rd = rng_for(idx, S_DRAFT, b)
    rs = rng_for(idx, S_SPIKE, b)
    rx = rng_for(idx, S_TOKEN, b)
    ru = rng_for(idx, S_UACC, b)
    rr = rng_for(idx, S_USAMP, b)
    out = {}
    if spec.index == 4:
        G = spec.G
        t64 = rt.standard_normal((G, k + 1, V)) * 3.0
        t = round_logits(t64, spec.dtype)
        tv = as_f64(t, spec.dtype)
        x = rs.integers(0, V, size=(G, k)).astype(np.int32)
        forced = rs.choice(G, size=4, replace=False)
        for c in forced:
            j = int(rs.integers(1, k + 1))
            x[c, :j] = np.argmax(tv[c, :j], axis=-1)
        out.update(target=t, draft=None, draft_tokens=x,
                   u_accept=exact_uniforms(ru, k), u_sample=exact_uniforms(rr, 1))
        return out
    sigma_t = {0: 3.0, 1: 3.0, 2: 4.0, 3: 3.0}[idx]
    t64 = rt.standard_normal((k + 1, V)) * sigma_t
    if idx == 2:
        n_spike = V // 100
        for i in range(k + 1):
            t64[i, rs.choice(V, size=n_spike, replace=False)] += 10.0
    if idx == 3:
        sigma_d = rd.uniform(0.2, 3.0)
    else:
        sigma_d = {0: 0.5, 1: 1.0, 2: 1.5}[idx]
    d64 = t64[:k] + rd.standard_normal((k, V)) * sigma_d
    t = round_logits(t64, spec.dtype)
    d = round_logits(d64, spec.dtype)
    dv = as_f64(d, spec.dtype)
    x = gumbel_max(rx, dv, spec.tau)
    out.update(target=t, draft=d, draft_tokens=x,
               u_accept=exact_uniforms(ru, k), u_sample=exact_uniforms(rr, 1))
    if idx == 2:
        out["greedy_tokens"] = np.argmax(dv, axis=-1).astype(np.int32)
    return out


def make(index: int, seqs=None, threads: int | None = None) -> Batch:
    """Generate workload ``index`` (all sequences, or the listed subset)."""
    spec = SPECS[index]
    seqs = np.arange(spec.B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda b: _sequence(spec, int(b)), seqs))
    n = len(parts)

    def stack(key):
        if parts[0].get(key) is None:
            return None
        return np.stack([p[key] for p in parts])

    return Batch(spec=spec, target=stack("target"), draft=stack("draft"),
                 draft_tokens=stack("draft_tokens"), u_accept=stack("u_accept").reshape(n, -1),
                 u_sample=stack("u_sample").reshape(n), greedy_tokens=stack("greedy_tokens"),
                 seqs=seqs)


@dataclass
class RaggedBatch:
    """Packed ragged batch.  target: [n + B][V] (sequence b's k_b + 1 rows from
    row cu[b] + b); draft: [n][V] (from row cu[b]); draft_tokens, u_accept:
    [n]; cu: int32 [B + 1] cumulative draft lengths; u_sample: [B]."""
    spec: Spec
    k_max: int
    kb: np.ndarray
    cu: np.ndarray
    target: np.ndarray
    draft: np.ndarray
    draft_tokens: np.ndarray
    u_accept: np.ndarray
    u_sample: np.ndarray


def ragged_lengths(spec: Spec, seqs=None) -> np.ndarray:
    """k_b ~ U{1..k} per sequence, from the length stream."""
    seqs = np.arange(spec.B) if seqs is None else np.asarray(seqs, dtype=np.int64)
    return np.array([int(rng_for(spec.index, S_LEN, int(b)).integers(1, spec.k + 1))
                     for b in seqs], dtype=np.int64)


def ragged(batch: Batch) -> RaggedBatch:
    """Keep the first k_b draft positions of every sequence of a dense
    single-candidate batch (target rows 0..k_b, draft rows 0..k_b-1) and pack
    them.  Row k_b of the target is the row that follows the last kept draft
    token, so the packed batch is a valid verification input."""
    s = batch.spec
    if s.G != 1 or batch.draft is None:
        raise ValueError("ragged batches are built from single-candidate stochastic workloads")
    kb = ragged_lengths(s, batch.seqs)
    B = len(kb)
    cu = np.concatenate([[0], np.cumsum(kb)]).astype(np.int32)
    n = int(cu[-1])
    V = s.V
    target = np.empty((n + B, V), batch.target.dtype)
    draft = np.empty((n, V), batch.draft.dtype)
    x = np.empty(n, np.int32)
    ua = np.empty(n, np.float32)
    for b in range(B):
        k, d0 = int(kb[b]), int(cu[b])
        target[d0 + b:d0 + b + k + 1] = batch.target[b, :k + 1]
        draft[d0:d0 + k] = batch.draft[b, :k]
        x[d0:d0 + k] = batch.draft_tokens[b, :k]
        ua[d0:d0 + k] = batch.u_accept[b, :k]
    return RaggedBatch(spec=s, k_max=s.k, kb=kb, cu=cu, target=target, draft=draft,
                       draft_tokens=x, u_accept=ua, u_sample=batch.u_sample.copy())


# A fixed 64-node draft tree in the style of EAGLE's Top-K trees: level sizes
# 1, 8, 16, 16, 12, 8, 3; node i of a level hangs under node i mod m of the
# previous level (m nodes), so the earliest (most probable) nodes of a level
# carry the most children.
TREE_LEVELS = (1, 8, 16, 16, 12, 8, 3)


def tree_parents(levels=TREE_LEVELS) -> np.ndarray:
    par = [-1]
    prev = [0]
    for size in levels[1:]:
        cur = []
        for i in range(size):
            par.append(prev[i % len(prev)])
            cur.append(len(par) - 1)
        prev = cur
    return np.array(par, dtype=np.int32)


@dataclass
class TreeBatch:
    """target: [B][N][V] (row j: the target's output at node j); node_tokens,
    parents: int32 [B][N]."""
    V: int
    dtype: int
    target: np.ndarray
    node_tokens: np.ndarray
    parents: np.ndarray


def tree_batch(B: int = 32, V: int = 128256, dtype: int = BF16, follow: float = 0.8,
               seed: int = 10_005) -> TreeBatch:
    """B sequences with the fixed 64-node tree; target rows ~ N(0, 3^2)
    (seeded per sequence); the first child of every node carries the argmax of
    its parent's row with probability `follow` (a drafter whose top choice is
    often right), other children a uniform token."""
    par = tree_parents()
    N = len(par)
    first = np.zeros(N, bool)
    seen = set()
    for j in range(1, N):
        if par[j] not in seen:
            first[j] = True
            seen.add(par[j])

    def one(b):
        r = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(0, b)))
        t = round_logits(r.standard_normal((N, V)) * 3.0, dtype)
        g = np.argmax(as_f64(t, dtype), axis=-1)
        x = r.integers(0, V, size=N).astype(np.int32)
        follow_draw = r.random(N)
        for j in range(1, N):
            if first[j] and follow_draw[j] < follow:
                x[j] = g[par[j]]
        x[0] = -1
        return t, x

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(one, range(B)))
    return TreeBatch(V=V, dtype=dtype, target=np.stack([p[0] for p in parts]),
                     node_tokens=np.stack([p[1] for p in parts]),
                     parents=np.tile(par, (B, 1)))


def sample_rows(batch: Batch):
    """One row per sequence for plain sampling: target row 0 ([B][V]) and the
    sequence's sample uniform ([B])."""
    t = batch.target if batch.spec.G == 1 else batch.target[:, 0]
    return np.ascontiguousarray(t[:, 0]), batch.u_sample.copy()
