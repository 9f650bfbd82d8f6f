"""Comparison of another implementation's outputs with the oracle.

TEST INFRASTRUCTURE ONLY.  Takes plain numpy arrays (it never imports the
implementation under test) and applies the agreement rules:

* greedy: accept_len, tokens and best_cand must be identical;
* stochastic: walking the positions in order, a decision may differ from the
  oracle's only where the acceptance uniform lies within ``BAND`` of the
  oracle's threshold min(1, p/q); the oracle is then re-run with that
  decision forced, and the walk continues.  The extra token may differ only
  where the oracle's draw is within ``BAND`` of a cumulative-distribution
  breakpoint AND the uniform lies within ``BAND`` of the other token's own
  interval under the oracle's distribution.  Probabilities p_i(x_i), q_i(x_i)
  must agree to ``REL`` relative.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import svo

BAND = 1e-5
REL = 1e-5
ABS_FLOOR = 1e-30  # probabilities this small are compared absolutely


@dataclass
class Report:
    n: int = 0
    decision_band: int = 0   # decisions that differed inside the band
    token_band: int = 0      # extra tokens that differed inside the band
    max_rel_p: float = 0.0
    failures: list = field(default_factory=list)

    def ok(self) -> bool:
        return not self.failures

    def summary(self) -> str:
        return (f"{self.n} sequences, {self.decision_band} in-band decisions, "
                f"{self.token_band} in-band tokens, max rel p/q err {self.max_rel_p:.2e}, "
                f"{len(self.failures)} failures" +
                ("" if not self.failures else ": " + "; ".join(self.failures[:5])))


def compare_greedy(oracle_out: dict, accept_len, tokens, best_cand=None) -> Report:
    rep = Report(n=len(accept_len))
    a_o, t_o = oracle_out["accept_len"], oracle_out["tokens"]
    for b in range(len(accept_len)):
        if int(accept_len[b]) != int(a_o[b]) or not np.array_equal(tokens[b], t_o[b]):
            rep.failures.append(f"seq {b}: accept {accept_len[b]} vs {a_o[b]}, "
                                f"tokens {tokens[b].tolist()} vs {t_o[b].tolist()}")
        elif best_cand is not None and int(best_cand[b]) != int(oracle_out["best_cand"][b]):
            rep.failures.append(f"seq {b}: best_cand {best_cand[b]} vs {oracle_out['best_cand'][b]}")
    return rep


def compare_stochastic(target, draft, draft_tokens, u_accept, u_sample, *, B, k, V,
                       temperature, accept_len, tokens, px_qx=None, row_stride=None,
                       lib=None) -> Report:
    """target/draft/draft_tokens/uniforms: the exact inputs the implementation
    saw (host copies).  accept_len [B], tokens [B][k+1], px_qx [B][k][2] or
    None: its outputs."""
    lib = lib or svo.load()
    rs = V if row_stride is None else row_stride
    rep = Report(n=B)
    o = svo.verify_stochastic(target, draft, draft_tokens, u_accept, u_sample, B=B, k=k, V=V,
                              row_stride=rs, temperature=temperature, lib=lib)
    # probabilities of the draft tokens
    if px_qx is not None:
        for name, g, r in (("p", px_qx[..., 0], o["px"]), ("q", px_qx[..., 1], o["qx"])):
            g = g.astype(np.float64)
            err = np.abs(g - r)
            big = np.abs(r) > ABS_FLOOR
            rel = np.where(big, err / np.where(big, np.abs(r), 1.0), 0.0)
            bad = (rel > REL) | (~big & (err > ABS_FLOOR))
            if big.any():
                rep.max_rel_p = max(rep.max_rel_p, float(rel.max()))
            for (b, i) in zip(*np.nonzero(bad)):
                rep.failures.append(f"seq {b} pos {i}: {name} {g[b, i]!r} vs oracle {r[b, i]!r}")
    ua = np.asarray(u_accept, np.float32).reshape(B, k)
    us = np.asarray(u_sample, np.float32).reshape(B)
    x = np.asarray(draft_tokens, np.int32).reshape(B, k)
    tgt = np.ascontiguousarray(target).reshape(B, -1)
    drf = np.ascontiguousarray(draft).reshape(B, -1)
    for b in range(B):
        a_g = int(accept_len[b])
        a_o = int(o["accept_len"][b])
        px = o["px"][b].copy()
        qx = o["qx"][b].copy()
        cur = {"a": a_o, "tokens": o["tokens"][b].copy(), "lo": o["cdf_lo"][b], "hi": o["cdf_hi"][b]}
        force = np.zeros(k, np.int8)
        ok = True
        # walk decisions
        for i in range(k + 1):
            if i == k:
                break
            g_acc = i < a_g
            o_acc = i < cur["a"]
            if i > min(a_g, cur["a"]):
                break
            if g_acc == o_acc:
                if not g_acc:
                    break
                continue
            thr = min(1.0, px[i] / qx[i]) if qx[i] > 0 else (1.0 if px[i] > 0 else 0.0)
            if abs(float(ua[b, i]) - thr) >= BAND:
                rep.failures.append(f"seq {b} pos {i}: decision {'accept' if g_acc else 'reject'} "
                                    f"vs oracle, u={ua[b, i]!r} threshold={thr!r}")
                ok = False
                break
            rep.decision_band += 1
            force[i] = svo.FORCE_ACCEPT if g_acc else svo.FORCE_REJECT
            r = svo.verify_stochastic(tgt[b], drf[b], x[b:b + 1], ua[b:b + 1], us[b:b + 1],
                                      B=1, k=k, V=V, row_stride=rs, temperature=temperature,
                                      force=force[None, :], lib=lib)
            cur = {"a": int(r["accept_len"][0]), "tokens": r["tokens"][0].copy(),
                   "lo": r["cdf_lo"][0], "hi": r["cdf_hi"][0]}
        if not ok:
            continue
        if a_g != cur["a"]:
            rep.failures.append(f"seq {b}: accept_len {a_g} vs oracle {cur['a']}")
            continue
        tg = np.asarray(tokens[b])
        to = cur["tokens"]
        if np.array_equal(tg, to):
            continue
        # only the extra token may differ, and only inside the band
        same_rest = np.array_equal(np.delete(tg, a_g), np.delete(to, a_g))
        yg = int(tg[a_g])
        r_ = float(us[b])
        margin = min(r_ - cur["lo"], cur["hi"] - r_)
        inside = False
        if 0 <= yg < V:
            lo_g, hi_g = svo.emit_cdf(tgt[b], drf[b], b=0, k=k, V=V, a=a_g, y=yg, row_stride=rs,
                                      temperature=temperature, lib=lib)
            inside = (lo_g - BAND) <= r_ < (hi_g + BAND)
        if same_rest and margin < BAND and inside:
            rep.token_band += 1
        else:
            rep.failures.append(f"seq {b}: tokens {tg.tolist()} vs oracle {to.tolist()} "
                                f"(r={r_!r}, oracle cell [{cur['lo']!r}, {cur['hi']!r}))")
    return rep


def _sample_cell(row, *, V, temperature, y, lib):
    """Cumulative probability (before, through) token y under softmax(row/T).
    The oracle's bonus-token distribution of a one-draft sequence whose two
    target rows are both `row` is exactly that softmax, so its own CDF
    routine gives the cell."""
    t2 = np.ascontiguousarray(np.stack([row[:V], row[:V]]))
    d1 = np.ascontiguousarray(row[None, :V])
    return svo.emit_cdf(t2, d1, b=0, k=1, V=V, a=1, y=y, temperature=temperature, lib=lib)


def compare_sample(logits, u, *, B, V, temperature, tokens, greedy=False, row_stride=None,
                   lib=None) -> Report:
    """Plain sampling, one token per row.  Greedy: identical.  Otherwise the
    token may differ from the oracle's only where u lies within BAND of the
    oracle's cell boundary AND within BAND of the other token's own cell."""
    lib = lib or svo.load()
    rs = V if row_stride is None else row_stride
    rep = Report(n=B)
    rows = np.ascontiguousarray(logits).reshape(B, -1)[:, :rs]
    y_o = svo.sample(rows, u, B=B, V=V, row_stride=rs, temperature=temperature, greedy=greedy,
                     lib=lib)
    for b in range(B):
        yg, yo = int(tokens[b]), int(y_o[b])
        if yg == yo:
            continue
        if greedy or not (0 <= yg < V):
            rep.failures.append(f"row {b}: token {yg} vs oracle {yo}")
            continue
        r_ = float(np.float32(u[b]))
        lo_o, hi_o = _sample_cell(rows[b], V=V, temperature=temperature, y=yo, lib=lib)
        lo_g, hi_g = _sample_cell(rows[b], V=V, temperature=temperature, y=yg, lib=lib)
        if min(r_ - lo_o, hi_o - r_) < BAND and (lo_g - BAND) <= r_ < (hi_g + BAND):
            rep.token_band += 1
        else:
            rep.failures.append(f"row {b}: token {yg} vs oracle {yo} (u={r_!r}, oracle cell "
                                f"[{lo_o!r}, {hi_o!r}), other cell [{lo_g!r}, {hi_g!r}))")
    return rep


def compare_stochastic_ragged(target, draft, draft_tokens, cu, u_accept, u_sample, *, k_max, V,
                              temperature, accept_len, tokens, px_qx=None, row_stride=None,
                              lib=None) -> Report:
    """Ragged batch: sequence b (k_b = cu[b+1] - cu[b] draft tokens, target
    rows from cu[b] + b, draft rows from cu[b]) is compared as a batch of one
    under the dense rules, or as plain sampling when k_b = 0; token slots past
    k_b must hold -1.  px_qx: [cu[B]][2] or None."""
    lib = lib or svo.load()
    rs = V if row_stride is None else row_stride
    cu = np.asarray(cu, np.int64).reshape(-1)
    B = cu.size - 1
    tgt = np.ascontiguousarray(target).reshape(-1, rs)
    drf = np.ascontiguousarray(draft).reshape(-1, rs) if cu[-1] > 0 else None
    x = np.asarray(draft_tokens, np.int32).reshape(-1)
    ua = np.asarray(u_accept, np.float32).reshape(-1)
    us = np.asarray(u_sample, np.float32).reshape(-1)
    rep = Report(n=B)
    for b in range(B):
        d0, kb = int(cu[b]), int(cu[b + 1] - cu[b])
        t0 = d0 + b
        tok = np.asarray(tokens[b])
        if np.any(tok[kb + 1:] != -1):
            rep.failures.append(f"seq {b}: slots past k_b={kb} not -1: {tok.tolist()}")
            continue
        if kb == 0:
            if int(accept_len[b]) != 0:
                rep.failures.append(f"seq {b}: accept_len {accept_len[b]} with no drafts")
                continue
            r = compare_sample(tgt[t0:t0 + 1], us[b:b + 1], B=1, V=V, temperature=temperature,
                               tokens=tok[:1], row_stride=rs, lib=lib)
        else:
            pq = None if px_qx is None else np.asarray(px_qx)[d0:d0 + kb][None]
            r = compare_stochastic(tgt[t0:t0 + kb + 1], drf[d0:d0 + kb], x[None, d0:d0 + kb],
                                   ua[None, d0:d0 + kb], us[b:b + 1], B=1, k=kb, V=V,
                                   temperature=temperature, accept_len=accept_len[b:b + 1],
                                   tokens=tok[None, :kb + 1], px_qx=pq, row_stride=rs, lib=lib)
        rep.decision_band += r.decision_band
        rep.token_band += r.token_band
        rep.max_rel_p = max(rep.max_rel_p, r.max_rel_p)
        rep.failures += [f"seq {b}: " + f for f in r.failures]
    return rep


def compare_greedy_ragged(oracle_out: dict, accept_len, tokens) -> Report:
    """Ragged greedy: identical accept lengths and token rows."""
    return compare_greedy(oracle_out, accept_len, tokens)
