"""ctypes front end of the float64 CPU oracle (``svo.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The oracle shares no code with the GPU
library; it is compiled from ``svo.c`` with the host C compiler.

Arrays are numpy arrays.  Logits are ``float32`` or raw bfloat16 bit patterns
(``uint16``), shaped ``[rows, row_stride]`` or anything that flattens to the
row layouts documented in ``svo.h``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svo.c")
_LIB_PATH = os.path.join(_HERE, "libsvo.so")

F32 = 0
BF16 = 1
FORCE_NONE = 0
FORCE_ACCEPT = 1
FORCE_REJECT = 2

_lib = None


def build(out_path: str = _LIB_PATH, src: str = _SRC, extra_flags=()) -> str:
    """Compile the oracle into a shared library (always recompiles)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-Wextra", "-fopenmp", "-shared",
           "-fPIC", *extra_flags, src, "-o", out_path, "-lm"]
    subprocess.run(cmd, check=True, cwd=_HERE)
    return out_path


def _bind(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.svo_verify_stochastic.argtypes = [P, P, P, P, P, I, I, I, ctypes.c_int64, I,
                                          ctypes.c_double, P, P, P, P, P, P, P]
    lib.svo_verify_stochastic.restype = I
    lib.svo_emit_cdf.argtypes = [P, P, I, I, I, ctypes.c_int64, I, ctypes.c_double,
                                 I, I, P, P]
    lib.svo_emit_cdf.restype = I
    lib.svo_verify_greedy.argtypes = [P, P, I, I, I, I, ctypes.c_int64, I, P, P, P, P]
    lib.svo_verify_greedy.restype = I
    lib.svo_verify_stochastic_ragged.argtypes = [P, P, P, P, P, P, I, I, I, ctypes.c_int64, I,
                                                 ctypes.c_double, P, P, P, P]
    lib.svo_verify_stochastic_ragged.restype = I
    lib.svo_verify_greedy_ragged.argtypes = [P, P, P, I, I, I, ctypes.c_int64, I, P, P]
    lib.svo_verify_greedy_ragged.restype = I
    lib.svo_sample.argtypes = [P, P, I, I, ctypes.c_int64, I, ctypes.c_double, I, P]
    lib.svo_sample.restype = I
    lib.svo_verify_greedy_tree.argtypes = [P, P, P, I, I, I, ctypes.c_int64, I, P, P, P]
    lib.svo_verify_greedy_tree.restype = I
    lib.svo_commit.argtypes = [P, P, I, I, P, P, ctypes.c_int64, I, P, ctypes.c_int64]
    lib.svo_commit.restype = I
    lib.svo_num_threads.argtypes = []
    lib.svo_num_threads.restype = I
    lib.svo_set_num_threads.argtypes = [I]
    lib.svo_set_num_threads.restype = None
    return lib


def load(path: str | None = None):
    """Load the oracle library (building it first only if it is absent)."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        _lib = _bind(ctypes.CDLL(_LIB_PATH))
    return _lib


def _ptr(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"logits must be float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def verify_stochastic(target, draft, draft_tokens, u_accept, u_sample, *, B, k, V,
                      row_stride=None, temperature=1.0, force=None, lib=None):
    """Run the oracle's stochastic verification.  Returns a dict of numpy arrays:
    accept_len [B], tokens [B][k+1], px [B][k], qx [B][k], cdf_lo [B], cdf_hi [B]."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    dt = _dtype_code(target)
    assert _dtype_code(draft) == dt
    row_stride = V if row_stride is None else int(row_stride)
    assert target.size >= B * (k + 1) * row_stride and draft.size >= B * k * row_stride
    x = _c(draft_tokens, np.int32).reshape(-1)
    ua = _c(u_accept, np.float32).reshape(-1)
    us = _c(u_sample, np.float32).reshape(-1)
    assert x.size == B * k and ua.size == B * k and us.size == B
    f = None if force is None else _c(force, np.int8).reshape(-1)
    out = dict(accept_len=np.zeros(B, np.int32), tokens=np.zeros((B, k + 1), np.int32),
               px=np.zeros((B, k)), qx=np.zeros((B, k)), cdf_lo=np.zeros(B),
               cdf_hi=np.zeros(B))
    rc = lib.svo_verify_stochastic(_ptr(target), _ptr(draft), _ptr(x), _ptr(ua), _ptr(us),
                                   B, k, V, row_stride, dt, float(temperature), _ptr(f),
                                   _ptr(out["accept_len"]), _ptr(out["tokens"]),
                                   _ptr(out["px"]), _ptr(out["qx"]), _ptr(out["cdf_lo"]),
                                   _ptr(out["cdf_hi"]))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def emit_cdf(target, draft, *, b, k, V, a, y, row_stride=None, temperature=1.0, lib=None):
    """Cumulative probability (before, through) token y under the distribution the
    extra token of sequence b is drawn from when the first rejection is at a."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    dt = _dtype_code(target)
    row_stride = V if row_stride is None else int(row_stride)
    lo = ctypes.c_double()
    hi = ctypes.c_double()
    rc = lib.svo_emit_cdf(_ptr(target), _ptr(draft), int(b), k, V, row_stride, dt,
                          float(temperature), int(a), int(y), ctypes.byref(lo),
                          ctypes.byref(hi))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return lo.value, hi.value


def verify_greedy(target, draft_tokens, *, B, G=1, k, V, row_stride=None, lib=None):
    """Run the oracle's greedy verification.  Returns accept_len [B],
    tokens [B][k+1], best_cand [B], cand_accept [B][G]."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    dt = _dtype_code(target)
    row_stride = V if row_stride is None else int(row_stride)
    assert target.size >= B * G * (k + 1) * row_stride
    x = _c(draft_tokens, np.int32).reshape(-1)
    assert x.size == B * G * k
    out = dict(accept_len=np.zeros(B, np.int32), tokens=np.zeros((B, k + 1), np.int32),
               best_cand=np.zeros(B, np.int32), cand_accept=np.zeros((B, G), np.int32))
    rc = lib.svo_verify_greedy(_ptr(target), _ptr(x), B, G, k, V, row_stride, dt,
                               _ptr(out["accept_len"]), _ptr(out["tokens"]),
                               _ptr(out["best_cand"]), _ptr(out["cand_accept"]))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def verify_stochastic_ragged(target, draft, draft_tokens, cu, u_accept, u_sample, *, k_max, V,
                             row_stride=None, temperature=1.0, lib=None):
    """Ragged stochastic verification (see svo.h).  cu: int32 [B+1].  Returns
    accept_len [B], tokens [B][k_max+1], px, qx [cu[B]]."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    draft = np.ascontiguousarray(draft)
    dt = _dtype_code(target)
    row_stride = V if row_stride is None else int(row_stride)
    cu = _c(cu, np.int32).reshape(-1)
    B = cu.size - 1
    n = int(cu[-1])
    assert target.size >= (n + B) * row_stride and draft.size >= n * row_stride
    x = _c(draft_tokens, np.int32).reshape(-1)
    ua = _c(u_accept, np.float32).reshape(-1)
    us = _c(u_sample, np.float32).reshape(-1)
    assert x.size >= n and ua.size >= n and us.size == B
    if n == 0:  # keep every pointer valid
        x, ua = np.zeros(1, np.int32), np.zeros(1, np.float32)
    out = dict(accept_len=np.zeros(B, np.int32), tokens=np.zeros((B, k_max + 1), np.int32),
               px=np.zeros(max(n, 1)), qx=np.zeros(max(n, 1)))
    d = draft if draft.size else np.zeros(1, draft.dtype)
    rc = lib.svo_verify_stochastic_ragged(_ptr(target), _ptr(d), _ptr(x), _ptr(cu), _ptr(ua),
                                          _ptr(us), B, k_max, V, row_stride, dt,
                                          float(temperature), _ptr(out["accept_len"]),
                                          _ptr(out["tokens"]), _ptr(out["px"]), _ptr(out["qx"]))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    out["px"], out["qx"] = out["px"][:n], out["qx"][:n]
    return out


def verify_greedy_ragged(target, draft_tokens, cu, *, k_max, V, row_stride=None, lib=None):
    """Ragged greedy verification (see svo.h).  Returns accept_len [B], tokens
    [B][k_max+1]."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    dt = _dtype_code(target)
    row_stride = V if row_stride is None else int(row_stride)
    cu = _c(cu, np.int32).reshape(-1)
    B = cu.size - 1
    x = _c(draft_tokens, np.int32).reshape(-1)
    if x.size == 0:
        x = np.zeros(1, np.int32)
    out = dict(accept_len=np.zeros(B, np.int32), tokens=np.zeros((B, k_max + 1), np.int32))
    rc = lib.svo_verify_greedy_ragged(_ptr(target), _ptr(x), _ptr(cu), B, k_max, V, row_stride,
                                      dt, _ptr(out["accept_len"]), _ptr(out["tokens"]))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def sample(logits, u, *, B, V, row_stride=None, temperature=1.0, greedy=False, lib=None):
    """Plain sampling of one token per row (see svo.h).  Returns int32 [B]."""
    lib = lib or load()
    logits = np.ascontiguousarray(logits)
    dt = _dtype_code(logits)
    row_stride = V if row_stride is None else int(row_stride)
    uu = None if u is None else _c(u, np.float32).reshape(-1)
    out = np.zeros(B, np.int32)
    rc = lib.svo_sample(_ptr(logits), _ptr(uu), B, V, row_stride, dt, float(temperature),
                        1 if greedy else 0, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def verify_greedy_tree(target, node_tokens, parents, *, B, N, V, row_stride=None, lib=None):
    """Greedy tree verification (see svo.h).  Returns accept_len [B], tokens
    [B][N], path [B][N]."""
    lib = lib or load()
    target = np.ascontiguousarray(target)
    dt = _dtype_code(target)
    row_stride = V if row_stride is None else int(row_stride)
    assert target.size >= B * N * row_stride
    x = _c(node_tokens, np.int32).reshape(-1)
    par = _c(parents, np.int32).reshape(-1)
    assert x.size == B * N and par.size == B * N
    out = dict(accept_len=np.zeros(B, np.int32), tokens=np.zeros((B, N), np.int32),
               path=np.zeros((B, N), np.int32))
    rc = lib.svo_verify_greedy_tree(_ptr(target), _ptr(x), _ptr(par), B, N, V, row_stride, dt,
                                    _ptr(out["accept_len"]), _ptr(out["tokens"]),
                                    _ptr(out["path"]))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def commit(accept_len, tokens, seq_len, history, *, capacity=None, next_stride=1, lib=None):
    """Commit of a verified step (see svo.h).  seq_len [B] and history
    [B][stride] are updated in place copies; returns (seq_len, history,
    next_token [B * next_stride] with the tokens at multiples of next_stride)."""
    lib = lib or load()
    a = _c(accept_len, np.int32).reshape(-1)
    B = a.size
    t = _c(tokens, np.int32).reshape(B, -1)
    W = t.shape[1]
    sl = np.array(seq_len, dtype=np.int32).reshape(-1).copy()
    h = np.array(history, dtype=np.int32).reshape(B, -1).copy()
    stride = h.shape[1]
    capacity = stride if capacity is None else int(capacity)
    nxt = np.full(max(B * next_stride, 1), -7, np.int32)
    rc = lib.svo_commit(_ptr(a), _ptr(t), B, W, _ptr(sl), _ptr(h), stride, capacity, _ptr(nxt),
                        next_stride)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return sl, h, nxt


def num_threads(lib=None) -> int:
    return (lib or load()).svo_num_threads()


def set_num_threads(n: int, lib=None) -> None:
    """Threads the oracle's OpenMP loops use from now on (timing only)."""
    (lib or load()).svo_set_num_threads(int(n))
