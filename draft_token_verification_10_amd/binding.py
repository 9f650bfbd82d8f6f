"""Thin ctypes binding of libspecverify on torch ROCm tensors.

Argument marshalling only: shapes and strides are read from the tensors,
pointers and the current HIP stream are passed to the C entry points of the
same names, and the status code is turned into an exception.  Every step of
the verification runs in the library's HIP kernels; there is no fallback.
If ``libspecverify.so`` has not been built, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os

import torch

from .build import LIB_PATH

SV_OK = 0
SV_DTYPE_F32 = 0
SV_DTYPE_BF16 = 1
SV_MAX_K = 64
SV_MAX_ROWS_PER_SEQ = 1024
SV_ERR_SCRATCH = -7
SV_SCRATCH_BYTES = 8 << 20

_lib = None


def load(path: str | None = None):
    """Load libspecverify.so (raises OSError when it is missing)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise OSError(f"{path} is missing: build it with __graft_entry__.build() "
                      "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.sv_verify_stochastic.argtypes = [P, P, P, P, P, I, I, I, I64, I, ctypes.c_float,
                                         P, P, P, P, SZ, P]
    lib.sv_verify_stochastic.restype = I
    lib.sv_verify_greedy.argtypes = [P, P, I, I, I, I, I64, I, P, P, P, P, SZ, P]
    lib.sv_verify_greedy.restype = I
    lib.sv_verify_stochastic_ragged.argtypes = [P, P, P, P, I, P, P, I, I, I, I64, I,
                                                ctypes.c_float, P, P, P, P, SZ, P]
    lib.sv_verify_stochastic_ragged.restype = I
    lib.sv_verify_greedy_ragged.argtypes = [P, P, P, I, I, I, I, I64, I, P, P, P, SZ, P]
    lib.sv_verify_greedy_ragged.restype = I
    lib.sv_sample.argtypes = [P, P, I, I, I64, I, ctypes.c_float, I, P, P, SZ, P]
    lib.sv_sample.restype = I
    lib.sv_verify_greedy_tree.argtypes = [P, P, P, I, I, I, I64, I, P, P, P, P, SZ, P]
    lib.sv_verify_greedy_tree.restype = I
    lib.sv_commit.argtypes = [P, P, I, I, P, P, I64, I, P, I64, P]
    lib.sv_commit.restype = I
    lib.sv_workspace_bytes.argtypes = [I, I, I, I]
    lib.sv_workspace_bytes.restype = SZ
    lib.sv_status_string.argtypes = [I]
    lib.sv_status_string.restype = ctypes.c_char_p
    lib.sv_stream_read.argtypes = [P, SZ, I, P, P]
    lib.sv_stream_read.restype = I
    lib.sv_verify_stochastic_noalloc.argtypes = [P, P, P, P, P, I, I, I, I64, I, ctypes.c_float,
                                                 P, P, P, P]
    lib.sv_verify_stochastic_noalloc.restype = I
    if path == LIB_PATH:
        _lib = lib
    return lib


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(f"libspecverify status {status}: {sv_status_string(status)}")


def sv_status_string(status: int) -> str:
    return load().sv_status_string(int(status)).decode()


def sv_workspace_bytes(B: int, G: int, k: int, V: int) -> int:
    return int(load().sv_workspace_bytes(int(B), int(G), int(k), int(V)))


# One cached workspace per (device, stream), grown on demand.  Its contents
# never matter between calls.
_workspaces: dict = {}


def workspace_for(nbytes: int, device: torch.device, stream: int):
    """The cached workspace of `stream`, at least `nbytes` long.  It is
    allocated on `stream` itself, so torch's caching allocator only ever
    reuses its memory -- or that of the smaller buffer it replaces -- for
    work ordered after the calls already queued on that stream."""
    if nbytes == 0:
        return None
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        if stream == torch.cuda.current_stream(device).cuda_stream:
            ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        else:
            with torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)):
                ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _ws_bytes(ws) -> int:
    return 0 if ws is None else ws.numel() * ws.element_size()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return SV_DTYPE_BF16
    raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _row_stride(t: torch.Tensor) -> int:
    """Element distance between consecutive logit rows; the rows of all
    leading dimensions must be evenly spaced."""
    if t.stride(-1) != 1:
        raise ValueError("logit rows must be contiguous along the vocabulary")
    for i in range(t.dim() - 2):
        if t.size(i) > 1 and t.stride(i) != t.stride(i + 1) * t.size(i + 1):
            raise ValueError("logit rows must be evenly spaced")
    return int(t.stride(-2)) if t.dim() >= 2 else int(t.size(-1))


def _dev(t: torch.Tensor) -> None:
    if not t.is_cuda:
        raise ValueError("all tensors must live on the GPU")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_i32(t, shape, name):
    _dev(t)
    if t.dtype != torch.int32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 tensor of shape {tuple(shape)}")


def _check_f32(t, shape, name):
    _dev(t)
    if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous float32 tensor of shape {tuple(shape)}")


def sv_verify_stochastic(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                         draft_tokens: torch.Tensor, u_accept: torch.Tensor,
                         u_sample: torch.Tensor, temperature: float = 1.0, *,
                         accept_len: torch.Tensor | None = None,
                         tokens: torch.Tensor | None = None,
                         dbg_px_qx: torch.Tensor | None = None,
                         workspace: torch.Tensor | None = None, stream=None):
    """Stochastic verification.  target_logits [B][k+1][V], draft_logits
    [B][k][V] (float32 or bfloat16; rows may be padded views), draft_tokens
    int32 [B][k], u_accept float32 [B][k], u_sample float32 [B].  Returns
    (accept_len int32 [B], tokens int32 [B][k+1]), written asynchronously on
    the current stream (or ``stream``)."""
    _dev(target_logits)
    _dev(draft_logits)
    B, k1, V = target_logits.shape
    k = k1 - 1
    if tuple(draft_logits.shape) != (B, k, V) or draft_logits.dtype != target_logits.dtype:
        raise ValueError("draft_logits must be [B][k][V] with the target's dtype")
    rs = _row_stride(target_logits)
    if B > 0 and _row_stride(draft_logits) != rs:
        raise ValueError("target and draft rows must share one row stride")
    _check_i32(draft_tokens, (B, k), "draft_tokens")
    _check_f32(u_accept, (B, k), "u_accept")
    _check_f32(u_sample, (B,), "u_sample")
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, k + 1), "tokens")
    if dbg_px_qx is not None:
        _check_f32(dbg_px_qx, (B, k, 2), "dbg_px_qx")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, 1, k, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_verify_stochastic(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
        _ptr(u_sample), B, k, V, rs, _dtype_code(target_logits), float(temperature),
        _ptr(accept_len), _ptr(tokens), _ptr(dbg_px_qx), _ptr(workspace), _ws_bytes(workspace),
        ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens


def sv_verify_stochastic_noalloc(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                 draft_tokens: torch.Tensor, u_accept: torch.Tensor,
                                 u_sample: torch.Tensor, temperature: float = 1.0, *,
                                 accept_len: torch.Tensor, tokens: torch.Tensor,
                                 dbg_px_qx: torch.Tensor | None = None, stream=None):
    """sv_verify_stochastic with the library's own per-GPU scratch buffer in
    place of a workspace: the call allocates nothing, so the outputs must be
    passed in.  Same shapes and results as sv_verify_stochastic."""
    _dev(target_logits)
    _dev(draft_logits)
    B, k1, V = target_logits.shape
    k = k1 - 1
    if tuple(draft_logits.shape) != (B, k, V) or draft_logits.dtype != target_logits.dtype:
        raise ValueError("draft_logits must be [B][k][V] with the target's dtype")
    rs = _row_stride(target_logits)
    if B > 0 and _row_stride(draft_logits) != rs:
        raise ValueError("target and draft rows must share one row stride")
    _check_i32(draft_tokens, (B, k), "draft_tokens")
    _check_f32(u_accept, (B, k), "u_accept")
    _check_f32(u_sample, (B,), "u_sample")
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, k + 1), "tokens")
    if dbg_px_qx is not None:
        _check_f32(dbg_px_qx, (B, k, 2), "dbg_px_qx")
    s = stream if stream is not None else torch.cuda.current_stream(target_logits.device).cuda_stream
    st = load().sv_verify_stochastic_noalloc(
        _ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), _ptr(u_accept),
        _ptr(u_sample), B, k, V, rs, _dtype_code(target_logits), float(temperature),
        _ptr(accept_len), _ptr(tokens), _ptr(dbg_px_qx), ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens


def sv_verify_greedy(target_logits: torch.Tensor, draft_tokens: torch.Tensor, *,
                     accept_len: torch.Tensor | None = None,
                     tokens: torch.Tensor | None = None,
                     best_cand: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None, stream=None):
    """Greedy verification.  target_logits [B][k+1][V] with draft_tokens
    [B][k], or [B][G][k+1][V] with [B][G][k] for G candidates.  Returns
    (accept_len [B], tokens [B][k+1], best_cand [B])."""
    _dev(target_logits)
    if target_logits.dim() == 3:
        B, k1, V = target_logits.shape
        G = 1
    else:
        B, G, k1, V = target_logits.shape
    k = k1 - 1
    rs = _row_stride(target_logits)
    _check_i32(draft_tokens, (B, k) if target_logits.dim() == 3 else (B, G, k), "draft_tokens")
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, k + 1), dtype=torch.int32, device=dev)
    if best_cand is None:
        best_cand = torch.empty(B, dtype=torch.int32, device=dev)
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, k + 1), "tokens")
    _check_i32(best_cand, (B,), "best_cand")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, G, k, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_verify_greedy(
        _ptr(target_logits), _ptr(draft_tokens), B, G, k, V, rs, _dtype_code(target_logits),
        _ptr(accept_len), _ptr(tokens), _ptr(best_cand), _ptr(workspace), _ws_bytes(workspace),
        ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens, best_cand


def _rows_2d(t: torch.Tensor, name: str):
    if t.dim() != 2:
        raise ValueError(f"{name} must be a [rows][V] tensor")
    return t.shape[0], t.shape[1], _row_stride(t)


def sv_verify_stochastic_ragged(target_logits: torch.Tensor, draft_logits: torch.Tensor,
                                draft_tokens: torch.Tensor, cu_draft_len: torch.Tensor,
                                u_accept: torch.Tensor, u_sample: torch.Tensor, k_max: int,
                                temperature: float = 1.0, *, total_draft: int | None = None,
                                accept_len=None, tokens=None, dbg_px_qx=None, workspace=None,
                                stream=None):
    """Ragged stochastic verification.  target_logits [total+B][V] and
    draft_logits [total][V] packed rows, draft_tokens int32 [total], cu_draft_len
    int32 [B+1] (device), u_accept float32 [total], u_sample float32 [B].
    total_draft defaults to draft_tokens' length.  Returns (accept_len [B],
    tokens [B][k_max+1])."""
    _dev(target_logits)
    nt, V, rs = _rows_2d(target_logits, "target_logits")
    B = cu_draft_len.numel() - 1
    total = int(draft_tokens.numel()) if total_draft is None else int(total_draft)
    if nt < total + B:
        raise ValueError("target_logits needs total_draft + B rows")
    _check_i32(cu_draft_len, (B + 1,), "cu_draft_len")
    if total > 0:
        _dev(draft_logits)
        nd, Vd, rsd = _rows_2d(draft_logits, "draft_logits")
        if Vd != V or rsd != rs or nd < total or draft_logits.dtype != target_logits.dtype:
            raise ValueError("draft_logits must be [total_draft][V] like the target rows")
        _check_i32(draft_tokens, (total,), "draft_tokens")
        _check_f32(u_accept, (total,), "u_accept")
    _check_f32(u_sample, (B,), "u_sample")
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, k_max + 1), "tokens")
    if dbg_px_qx is not None:
        _check_f32(dbg_px_qx, (total, 2), "dbg_px_qx")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, 1, k_max, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_verify_stochastic_ragged(
        _ptr(target_logits), _ptr(draft_logits if total > 0 else None),
        _ptr(draft_tokens if total > 0 else None), _ptr(cu_draft_len), total,
        _ptr(u_accept if total > 0 else None), _ptr(u_sample), B, k_max, V, rs,
        _dtype_code(target_logits), float(temperature), _ptr(accept_len), _ptr(tokens),
        _ptr(dbg_px_qx), _ptr(workspace), _ws_bytes(workspace), ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens


def sv_verify_greedy_ragged(target_logits: torch.Tensor, draft_tokens: torch.Tensor,
                            cu_draft_len: torch.Tensor, k_max: int, *,
                            total_draft: int | None = None, accept_len=None, tokens=None,
                            workspace=None, stream=None):
    """Ragged greedy verification (one candidate per sequence).  Returns
    (accept_len [B], tokens [B][k_max+1])."""
    _dev(target_logits)
    nt, V, rs = _rows_2d(target_logits, "target_logits")
    B = cu_draft_len.numel() - 1
    total = int(draft_tokens.numel()) if total_draft is None else int(total_draft)
    if nt < total + B:
        raise ValueError("target_logits needs total_draft + B rows")
    _check_i32(cu_draft_len, (B + 1,), "cu_draft_len")
    if total > 0:
        _check_i32(draft_tokens, (total,), "draft_tokens")
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, k_max + 1), dtype=torch.int32, device=dev)
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, k_max + 1), "tokens")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, 1, k_max, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_verify_greedy_ragged(
        _ptr(target_logits), _ptr(draft_tokens if total > 0 else None), _ptr(cu_draft_len),
        total, B, k_max, V, rs, _dtype_code(target_logits), _ptr(accept_len), _ptr(tokens),
        _ptr(workspace), _ws_bytes(workspace), ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens


def sv_sample(logits: torch.Tensor, u: torch.Tensor | None, temperature: float = 1.0, *,
              greedy: bool = False, tokens=None, workspace=None, stream=None):
    """One token per row of logits [B][V]: inverse CDF of softmax(row/T) at
    u[b], or the argmax when greedy.  Returns int32 [B]."""
    _dev(logits)
    B, V, rs = _rows_2d(logits, "logits")
    if not greedy:
        _check_f32(u, (B,), "u")
    dev = logits.device
    if tokens is None:
        tokens = torch.empty(B, dtype=torch.int32, device=dev)
    _check_i32(tokens, (B,), "tokens")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, 1, 0, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_sample(_ptr(logits), _ptr(None if greedy else u), B, V, rs,
                          _dtype_code(logits), float(temperature), 1 if greedy else 0,
                          _ptr(tokens), _ptr(workspace), _ws_bytes(workspace),
                          ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return tokens


def sv_verify_greedy_tree(target_logits: torch.Tensor, node_tokens: torch.Tensor,
                          parents: torch.Tensor, *, accept_len=None, tokens=None, path=None,
                          workspace=None, stream=None):
    """Greedy verification of one draft tree per sequence.  target_logits
    [B][N][V] (row j: the target's output at node j), node_tokens and parents
    int32 [B][N].  Returns (accept_len [B], tokens [B][N], path [B][N])."""
    _dev(target_logits)
    if target_logits.dim() != 3:
        raise ValueError("target_logits must be [B][N][V]")
    B, N, V = target_logits.shape
    rs = _row_stride(target_logits)
    _check_i32(node_tokens, (B, N), "node_tokens")
    _check_i32(parents, (B, N), "parents")
    dev = target_logits.device
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((B, N), dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty((B, N), dtype=torch.int32, device=dev)
    _check_i32(accept_len, (B,), "accept_len")
    _check_i32(tokens, (B, N), "tokens")
    _check_i32(path, (B, N), "path")
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    need = sv_workspace_bytes(B, N, 0, V) if B > 0 else 0
    if workspace is None:
        workspace = workspace_for(need, dev, s)
    st = load().sv_verify_greedy_tree(
        _ptr(target_logits), _ptr(node_tokens), _ptr(parents), B, N, V, rs,
        _dtype_code(target_logits), _ptr(accept_len), _ptr(tokens), _ptr(path), _ptr(workspace),
        _ws_bytes(workspace), ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return accept_len, tokens, path


def sv_commit(accept_len: torch.Tensor, tokens: torch.Tensor, seq_len: torch.Tensor,
              history: torch.Tensor, next_token: torch.Tensor, *, capacity: int | None = None,
              stream=None):
    """Commit a verified step on the GPU: append each sequence's emitted tokens
    to history [B][>= capacity] (int32, rows contiguous), advance seq_len [B]
    and write the last emitted token to next_token (a [B] int32 view whose
    elements may be strided, e.g. column 0 of the next step's input ids)."""
    _check_i32(accept_len, (accept_len.numel(),), "accept_len")
    B = accept_len.numel()
    if tokens.dim() != 2 or tokens.shape[0] != B:
        raise ValueError("tokens must be [B][W]")
    _check_i32(tokens, tuple(tokens.shape), "tokens")
    _check_i32(seq_len, (B,), "seq_len")
    _dev(history)
    if history.dtype != torch.int32 or history.dim() != 2 or history.shape[0] != B or \
            history.stride(1) != 1:
        raise ValueError("history must be an int32 [B][capacity] tensor with contiguous rows")
    _dev(next_token)
    if next_token.dtype != torch.int32 or next_token.dim() != 1 or next_token.numel() != B:
        raise ValueError("next_token must be an int32 [B] tensor")
    cap = history.shape[1] if capacity is None else int(capacity)
    if cap > history.shape[1]:
        raise ValueError("capacity exceeds the history rows")
    hs = history.stride(0) if B > 1 else history.shape[1]
    ns = next_token.stride(0) if B > 1 else 1
    dev = accept_len.device
    s = stream if stream is not None else torch.cuda.current_stream(dev).cuda_stream
    st = load().sv_commit(_ptr(accept_len), _ptr(tokens), B, tokens.shape[1], _ptr(seq_len),
                          _ptr(history), hs, cap, _ptr(next_token), max(ns, 1),
                          ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
    return seq_len, history, next_token


def sv_stream_read(buf: torch.Tensor, blocks: int, out: torch.Tensor, stream=None) -> None:
    """Measurement aid: read the contiguous device tensor `buf` once with the
    logit stream's loads, `blocks` workgroups each reading one contiguous
    share; `out` (int32 [>= blocks] on the same device) receives one XOR
    checksum per workgroup."""
    _dev(buf)
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    if out.dtype != torch.int32 or out.numel() < blocks or out.device != buf.device:
        raise ValueError("out must be an int32 tensor of at least `blocks` words on buf's device")
    s = stream if stream is not None else torch.cuda.current_stream(buf.device).cuda_stream
    st = load().sv_stream_read(_ptr(buf), buf.numel() * buf.element_size(), int(blocks),
                               _ptr(out), ctypes.c_void_p(s))
    if st != SV_OK:
        raise SpecVerifyError(st)
