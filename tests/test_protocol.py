"""The agreement rules of oracle/protocol.py on outputs built on the CPU:
the oracle's own outputs pass, a planted wrong token or decision fails, and
a difference inside the 1e-5 band at a CDF breakpoint passes."""
import numpy as np

from oracle import protocol, svo
from tests.oracle_pins import ragged_batch, softmax64


def test_dense_own_output_passes_and_wrong_fails():
    rng = np.random.default_rng(5)
    B, k, V = 12, 4, 30
    t = (rng.standard_normal((B, k + 1, V)) * 2).astype(np.float32)
    d = (t[:, :k] + rng.standard_normal((B, k, V))).astype(np.float32)
    x = rng.integers(0, V, size=(B, k)).astype(np.int32)
    ua = rng.random((B, k)).astype(np.float32)
    us = rng.random(B).astype(np.float32)
    o = svo.verify_stochastic(t, d, x, ua, us, B=B, k=k, V=V)
    pq = np.stack([o["px"], o["qx"]], -1).astype(np.float32)
    kw = dict(B=B, k=k, V=V, temperature=1.0)
    assert protocol.compare_stochastic(t, d, x, ua, us, accept_len=o["accept_len"],
                                       tokens=o["tokens"], px_qx=pq, **kw).ok()
    a = o["accept_len"].copy()
    b = int(np.argmin(a))
    a[b] += 1
    assert not protocol.compare_stochastic(t, d, x, ua, us, accept_len=a, tokens=o["tokens"],
                                           **kw).ok()
    pq2 = pq.copy()
    pq2[0, 0, 0] *= 1.001
    assert not protocol.compare_stochastic(t, d, x, ua, us, accept_len=o["accept_len"],
                                           tokens=o["tokens"], px_qx=pq2, **kw).ok()


def test_ragged_own_output_passes_and_wrong_fails():
    rng = np.random.default_rng(6)
    kb, cu, t, d, x, ua, us = ragged_batch(rng, 25, 5, 40)
    o = svo.verify_stochastic_ragged(t, d, x, cu, ua, us, k_max=5, V=40)
    pq = np.stack([o["px"], o["qx"]], -1).astype(np.float32)
    kw = dict(k_max=5, V=40, temperature=1.0)
    assert protocol.compare_stochastic_ragged(t, d, x, cu, ua, us, accept_len=o["accept_len"],
                                              tokens=o["tokens"], px_qx=pq, **kw).ok()
    for b in (int(np.nonzero(kb == 0)[0][0]), int(np.nonzero(kb == 5)[0][0])):
        tok = o["tokens"].copy()
        j = int(o["accept_len"][b])
        tok[b, j] = (tok[b, j] + 1) % 40
        assert not protocol.compare_stochastic_ragged(t, d, x, cu, ua, us,
                                                      accept_len=o["accept_len"], tokens=tok,
                                                      **kw).ok()
    # a slot past k_b that is not -1
    b = int(np.nonzero(kb < 5)[0][0])
    tok = o["tokens"].copy()
    tok[b, 5] = 0
    assert not protocol.compare_stochastic_ragged(t, d, x, cu, ua, us, accept_len=o["accept_len"],
                                                  tokens=tok, **kw).ok()


def test_sample_band_at_breakpoint():
    V = 6
    row = np.log(np.array([0.25, 0.125, 0.125, 0.25, 0.125, 0.125], np.float64)).astype(np.float32)
    p = softmax64(row)
    c1 = float(np.cumsum(p)[0])  # breakpoint between tokens 0 and 1
    u_below = np.float32(np.nextafter(np.float32(c1), np.float32(0)))
    u = np.array([u_below, 0.6], np.float32)
    rows = np.stack([row, row])
    y = svo.sample(rows, u, B=2, V=V)
    assert y[0] == 0
    # token 1 for u just below the breakpoint: inside the band
    rep = protocol.compare_sample(rows, u, B=2, V=V, temperature=1.0,
                                  tokens=np.array([1, y[1]], np.int32))
    assert rep.ok() and rep.token_band == 1
    # a far token is not
    assert not protocol.compare_sample(rows, u, B=2, V=V, temperature=1.0,
                                       tokens=np.array([4, y[1]], np.int32)).ok()
    # greedy allows no difference
    ti = np.array([[0, 3, 3, 1]], np.float32)
    assert protocol.compare_sample(ti, None, B=1, V=4, temperature=1.0, greedy=True,
                                   tokens=np.array([1], np.int32)).ok()
    assert not protocol.compare_sample(ti, None, B=1, V=4, temperature=1.0, greedy=True,
                                       tokens=np.array([2], np.int32)).ok()
