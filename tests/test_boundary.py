"""The C ABI without a GPU: the library loads, exports what the header
declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

from draft_token_verification_10_amd import binding
from draft_token_verification_10_amd.build import INCLUDE, LIB_PATH

HEADER = os.path.join(INCLUDE, "specverify.h")

SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_TEMPERATURE, SV_ERR_WORKSPACE, SV_ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6
SV_ERR_SCRATCH = -7


HEADERS = sorted(os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE) if f.endswith(".h"))


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(sv_\w+)\s*\(", text))
    return sorted(names)


def header_constants():
    text = open(HEADER).read()
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(SV_\w+)\s+\(?(-?\d+)\)?", text)}


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        pytest.skip("libspecverify.so not built")
    # The checks below pass fake device addresses and rely on the host-side
    # argument checks refusing every call; they run where no GPU is visible,
    # so that a regression in a check can never launch on those addresses.
    import torch
    if torch.cuda.is_available():
        pytest.skip("host argument checks are exercised without a GPU")
    return binding.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == ["sv_commit", "sv_sample", "sv_status_string", "sv_stream_read",
                     "sv_verify_greedy", "sv_verify_greedy_ragged", "sv_verify_greedy_tree",
                     "sv_verify_stochastic", "sv_verify_stochastic_noalloc",
                     "sv_verify_stochastic_ragged", "sv_workspace_bytes"]
    for n in names:
        assert hasattr(lib, n), n


def test_header_constants_match_binding():
    c = header_constants()
    assert c["SV_OK"] == SV_OK and c["SV_ERR_NULL"] == SV_ERR_NULL
    assert c["SV_ERR_SHAPE"] == SV_ERR_SHAPE and c["SV_ERR_DTYPE"] == SV_ERR_DTYPE
    assert c["SV_ERR_TEMPERATURE"] == SV_ERR_TEMPERATURE
    assert c["SV_ERR_WORKSPACE"] == SV_ERR_WORKSPACE and c["SV_ERR_HIP"] == SV_ERR_HIP
    assert c["SV_DTYPE_F32"] == binding.SV_DTYPE_F32
    assert c["SV_DTYPE_BF16"] == binding.SV_DTYPE_BF16
    assert c["SV_MAX_K"] == binding.SV_MAX_K
    assert c["SV_MAX_ROWS_PER_SEQ"] == binding.SV_MAX_ROWS_PER_SEQ
    assert c["SV_ERR_SCRATCH"] == SV_ERR_SCRATCH == binding.SV_ERR_SCRATCH
    assert c["SV_SCRATCH_BYTES"] == binding.SV_SCRATCH_BYTES == 8 << 20


def test_status_strings(lib):
    seen = set()
    for st in (SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_TEMPERATURE,
               SV_ERR_WORKSPACE, SV_ERR_HIP, SV_ERR_SCRATCH):
        s = lib.sv_status_string(st).decode()
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert lib.sv_status_string(12345).decode() == "unknown status"


def test_workspace_bytes(lib):
    f = lib.sv_workspace_bytes
    assert f(0, 1, 1, 1) == 0 or f(0, 1, 1, 1) % 256 == 0
    for args in [(64, 1, 4, 128256), (1, 1, 4, 32000), (32, 16, 4, 32000), (191, 1, 8, 1000),
                 (256, 2, 8, 1000)]:
        n = f(*args)
        assert n > 0 and n % 8 == 0
    # one candidate and B >= 192: dense calls run one workgroup per sequence
    # with no scratch, but the bound also covers ragged calls with
    # diagnostics, which may take the row-split layout
    for args in [(192, 1, 8, 128256), (256, 1, 8, 128256), (512, 1, 3, 129280)]:
        assert f(*args) >= args[0] * (2 * args[2] + 1) * 8
    # ... and, for 128..1024 sequences with k >= 6, the capped early exit: a
    # flag per sequence, statistics for up to 16 slices per row, the draw's
    # tile sums; no such term for k < 6, below 128 or beyond 1024 sequences
    for B, k in [(128, 8), (160, 6), (192, 6), (256, 8), (1024, 64)]:
        assert f(B, 1, k, 128256) >= B * 4 + B * (2 * k + 1) * 16 * 8 + B * 257 * 4
    assert f(256, 1, 5, 128256) < 256 * 11 * 16 * 8
    assert f(1025, 1, 8, 128256) < 1025 * 17 * 16 * 8
    assert f(127, 1, 8, 128256) < 127 * 4 + 127 * 17 * 16 * 8 + 127 * 257 * 4
    # bad shapes
    for args in [(-1, 1, 1, 10), (1, 0, 1, 10), (1, 1, -1, 10), (1, 1, 1, 0), (1, 1, 65, 10),
                 (1, 600, 1, 10)]:
        assert f(*args) == 0
    # k = 0 (plain sampling) is a valid shape; the bound covers the sliced
    # layout's slices of at most about 16384 logits (8 for V = 128256)
    assert f(10, 1, 0, 1000) > 0
    assert f(256, 1, 0, 128256) >= 256 * 8 * 8
    # row-split: at least 8 bytes per row of every sequence
    for B in (1, 50, 100, 150, 191):
        assert f(B, 1, 8, 128256) >= B * 17 * 8
    assert f(32, 16, 4, 32000) >= 32 * 16 * 5 * 8


# Fake, well-aligned device addresses: the checks below fail before any
# pointer is used, so nothing is dereferenced or launched.
A = ctypes.c_void_p(1 << 20)
WS = ctypes.c_void_p(1 << 21)


def stoch(lib, **kw):
    args = dict(t=A, d=A, x=A, ua=A, us=A, B=2, k=3, V=100, rs=100, dtype=1, tau=1.0,
                al=A, tok=A, dbg=None, ws=WS, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_stochastic(args["t"], args["d"], args["x"], args["ua"], args["us"],
                                    args["B"], args["k"], args["V"], args["rs"], args["dtype"],
                                    args["tau"], args["al"], args["tok"], args["dbg"], args["ws"],
                                    args["wsb"], args["stream"])


def greedy(lib, **kw):
    args = dict(t=A, x=A, B=2, G=1, k=3, V=100, rs=100, dtype=0, al=A, tok=A, bc=None, ws=WS,
                wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_greedy(args["t"], args["x"], args["B"], args["G"], args["k"],
                                args["V"], args["rs"], args["dtype"], args["al"], args["tok"],
                                args["bc"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("field", ["t", "d", "x", "ua", "us", "al", "tok", "ws"])
def test_stochastic_null(lib, field):
    assert stoch(lib, **{field: None}) == SV_ERR_NULL


@pytest.mark.parametrize("field", ["t", "x", "al", "tok", "ws"])
def test_greedy_null(lib, field):
    assert greedy(lib, **{field: None}) == SV_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=-1), dict(k=-1), dict(k=65), dict(V=0), dict(rs=99),
                                dict(V=(1 << 28) + 1, rs=(1 << 28) + 1)])
def test_stochastic_shape(lib, kw):
    assert stoch(lib, **kw) == SV_ERR_SHAPE


@pytest.mark.parametrize("kw", [dict(B=-3), dict(G=0), dict(k=-2), dict(V=-5), dict(rs=10),
                                dict(G=300, k=3), dict(G=16, k=64)])
def test_greedy_shape(lib, kw):
    assert greedy(lib, **kw) == SV_ERR_SHAPE


def test_grid_too_large(lib):
    # the launch's thread count must fit in 32 bits: 2^25 row-split groups of
    # 256 threads, or 2^22 sequence-resident groups of 1024, are too many
    assert greedy(lib, B=1 << 21, G=2, k=7, V=10, rs=10) == SV_ERR_SHAPE
    assert greedy(lib, B=1 << 22, G=1, k=7, V=10, rs=10) == SV_ERR_SHAPE
    assert stoch(lib, B=1 << 22, k=7, V=10, rs=10) == SV_ERR_SHAPE


def test_dtype(lib):
    assert stoch(lib, dtype=2) == SV_ERR_DTYPE
    assert greedy(lib, dtype=-1) == SV_ERR_DTYPE


@pytest.mark.parametrize("tau", [0.0, -1.0, float("inf"), float("nan"), 1e-45])
def test_temperature(lib, tau):
    assert stoch(lib, tau=tau) == SV_ERR_TEMPERATURE


def test_workspace_checks(lib):
    need = lib.sv_workspace_bytes(2, 1, 3, 100)
    assert stoch(lib, wsb=need - 1) == SV_ERR_WORKSPACE
    assert stoch(lib, ws=ctypes.c_void_p((1 << 21) + 16)) == SV_ERR_WORKSPACE
    assert greedy(lib, wsb=8) == SV_ERR_WORKSPACE


def test_workspace_optional_without_scratch(lib):
    # B < 192 needs scratch
    assert stoch(lib, B=100, ws=None) == SV_ERR_NULL


def test_empty_batch_is_a_noop(lib):
    assert stoch(lib, B=0, t=None, d=None, x=None, ua=None, us=None, al=None, tok=None,
                 ws=None, wsb=0) == SV_OK
    assert greedy(lib, B=0, t=None, x=None, al=None, tok=None, ws=None, wsb=0) == SV_OK


def ragged(lib, **kw):
    args = dict(t=A, d=A, x=A, cu=A, total=10, ua=A, us=A, B=2, k=3, V=100, rs=100, dtype=1,
                tau=1.0, al=A, tok=A, dbg=None, ws=WS, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_stochastic_ragged(args["t"], args["d"], args["x"], args["cu"],
                                           args["total"], args["ua"], args["us"], args["B"],
                                           args["k"], args["V"], args["rs"], args["dtype"],
                                           args["tau"], args["al"], args["tok"], args["dbg"],
                                           args["ws"], args["wsb"], args["stream"])


def greedy_ragged(lib, **kw):
    args = dict(t=A, x=A, cu=A, total=10, B=2, k=3, V=100, rs=100, dtype=0, al=A, tok=A,
                ws=WS, wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_greedy_ragged(args["t"], args["x"], args["cu"], args["total"],
                                       args["B"], args["k"], args["V"], args["rs"],
                                       args["dtype"], args["al"], args["tok"], args["ws"],
                                       args["wsb"], args["stream"])


def sample(lib, **kw):
    args = dict(t=A, u=A, B=2, V=100, rs=100, dtype=1, tau=1.0, greedy=0, tok=A, ws=WS,
                wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_sample(args["t"], args["u"], args["B"], args["V"], args["rs"], args["dtype"],
                         args["tau"], args["greedy"], args["tok"], args["ws"], args["wsb"],
                         args["stream"])


@pytest.mark.parametrize("field", ["t", "d", "x", "cu", "ua", "us", "al", "tok", "ws"])
def test_ragged_null(lib, field):
    assert ragged(lib, **{field: None}) == SV_ERR_NULL


def test_ragged_without_drafts_needs_no_draft_buffers(lib):
    # total_draft == 0: draft logits, tokens and uniforms may be NULL; the
    # workspace check (too small) is the first to fail, before any launch
    assert ragged(lib, total=0, d=None, x=None, ua=None, wsb=8) == SV_ERR_WORKSPACE
    assert ragged(lib, total=0, d=None, x=None, ua=None, us=None) == SV_ERR_NULL


@pytest.mark.parametrize("kw", [dict(total=-1), dict(k=65), dict(k=-1), dict(B=-1),
                                dict(rs=50)])
def test_ragged_shape(lib, kw):
    assert ragged(lib, **kw) == SV_ERR_SHAPE


def test_ragged_other_checks(lib):
    assert ragged(lib, tau=0.0) == SV_ERR_TEMPERATURE
    assert ragged(lib, dtype=7) == SV_ERR_DTYPE
    assert ragged(lib, wsb=16) == SV_ERR_WORKSPACE
    assert ragged(lib, B=0, t=None, d=None, x=None, cu=None, ua=None, us=None, al=None,
                  tok=None, ws=None, wsb=0) == SV_OK


@pytest.mark.parametrize("field", ["t", "cu", "x", "al", "tok", "ws"])
def test_greedy_ragged_null(lib, field):
    assert greedy_ragged(lib, **{field: None}) == SV_ERR_NULL


def test_greedy_ragged_checks(lib):
    assert greedy_ragged(lib, total=-5) == SV_ERR_SHAPE
    assert greedy_ragged(lib, dtype=3) == SV_ERR_DTYPE
    assert greedy_ragged(lib, wsb=0) == SV_ERR_WORKSPACE


def test_sample_checks(lib):
    assert sample(lib, t=None) == SV_ERR_NULL
    assert sample(lib, u=None) == SV_ERR_NULL          # stochastic needs uniforms
    assert sample(lib, tok=None) == SV_ERR_NULL
    assert sample(lib, u=None, greedy=1, wsb=0) == SV_ERR_WORKSPACE  # greedy: u unused
    assert sample(lib, tau=-1.0) == SV_ERR_TEMPERATURE
    assert sample(lib, dtype=9) == SV_ERR_DTYPE
    assert sample(lib, V=0) == SV_ERR_SHAPE
    assert sample(lib, B=0, t=None, u=None, tok=None, ws=None, wsb=0) == SV_OK
    # the sliced layout (more than 512 rows, or rows too long for one pass)
    # needs the workspace: checked before any launch
    assert sample(lib, B=600, ws=None, wsb=0) == SV_ERR_NULL
    assert sample(lib, B=600, wsb=64) == SV_ERR_WORKSPACE
    assert sample(lib, V=100000, rs=100000, ws=None, wsb=0) == SV_ERR_NULL


def tree(lib, **kw):
    args = dict(t=A, x=A, par=A, B=2, N=5, V=100, rs=100, dtype=1, al=A, tok=A, path=A, ws=WS,
                wsb=1 << 30, stream=None)
    args.update(kw)
    return lib.sv_verify_greedy_tree(args["t"], args["x"], args["par"], args["B"], args["N"],
                                     args["V"], args["rs"], args["dtype"], args["al"],
                                     args["tok"], args["path"], args["ws"], args["wsb"],
                                     args["stream"])


def commit(lib, **kw):
    args = dict(al=A, tok=A, B=4, W=9, sl=A, h=A, hs=100, cap=100, nx=A, ns=1, stream=None)
    args.update(kw)
    return lib.sv_commit(args["al"], args["tok"], args["B"], args["W"], args["sl"], args["h"],
                         args["hs"], args["cap"], args["nx"], args["ns"], args["stream"])


@pytest.mark.parametrize("field", ["t", "x", "par", "al", "tok", "path", "ws"])
def test_tree_null(lib, field):
    assert tree(lib, **{field: None}) == SV_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=-1), dict(N=0), dict(N=1025), dict(V=0), dict(rs=99)])
def test_tree_shape(lib, kw):
    assert tree(lib, **kw) == SV_ERR_SHAPE


def test_tree_other_checks(lib):
    assert tree(lib, dtype=5) == SV_ERR_DTYPE
    assert tree(lib, wsb=0) == SV_ERR_WORKSPACE
    assert tree(lib, B=0, t=None, x=None, par=None, al=None, tok=None, path=None, ws=None,
                wsb=0) == SV_OK
    # the workspace bound for a tree: G = N nodes, k = 0
    assert lib.sv_workspace_bytes(256, 64, 0, 128256) >= 256 * 64 * 8
    assert lib.sv_workspace_bytes(300, 1, 0, 1000) > 0  # a root-only tree at a large batch


@pytest.mark.parametrize("field", ["al", "tok", "sl", "h", "nx"])
def test_commit_null(lib, field):
    assert commit(lib, **{field: None}) == SV_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=-1), dict(W=0), dict(cap=-1), dict(hs=50),
                                dict(ns=0)])
def test_commit_shape(lib, kw):
    assert commit(lib, **kw) == SV_ERR_SHAPE


def test_commit_empty(lib):
    assert commit(lib, B=0, al=None, tok=None, sl=None, h=None, nx=None) == SV_OK


def test_header_is_plain_c_and_links(tmp_path):
    """include/specverify.h compiles as C99 with warnings as errors, and a C
    program links against libspecverify and gets the documented statuses."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no host C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.dirname(LIB_PATH)
    exe = tmp_path / "abi_check"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(root, "include"), os.path.join(root, "tests", "c", "abi_check.c"),
                    "-L", libdir, "-lspecverify", f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr)


def test_stream_read_checks(lib):
    out = ctypes.c_void_p(1 << 22)
    assert lib.sv_stream_read(None, 0, 1, None, None) == SV_OK
    assert lib.sv_stream_read(None, 16, 1, out, None) == SV_ERR_NULL
    assert lib.sv_stream_read(A, 16, 1, None, None) == SV_ERR_NULL
    assert lib.sv_stream_read(A, 24, 1, out, None) == SV_ERR_SHAPE
    assert lib.sv_stream_read(ctypes.c_void_p((1 << 20) + 4), 16, 1, out, None) == SV_ERR_SHAPE
    for blocks in (0, -1, 65537):
        assert lib.sv_stream_read(A, 16, blocks, out, None) == SV_ERR_SHAPE
    assert lib.sv_stream_read(A, 1 << 32, 1, out, None) == SV_ERR_SHAPE  # share above 2 GiB


def test_noalloc_host_checks(lib):
    """sv_verify_stochastic_noalloc refuses, before touching any device, a
    shape whose workspace exceeds the library's own buffer, and passes every
    other bad argument to the checks of sv_verify_stochastic."""
    P = ctypes.c_void_p
    f = lib.sv_verify_stochastic_noalloc
    f.argtypes = [P, P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_int, ctypes.c_float, P, P, P, P]
    f.restype = ctypes.c_int
    fake = P(1 << 40)
    big = (1024, 64, 128256)
    assert lib.sv_workspace_bytes(big[0], 1, big[1], big[2]) > binding.SV_SCRATCH_BYTES
    assert f(fake, fake, fake, fake, fake, *big, big[2], 1, 1.0, fake, fake, None, None) == \
        SV_ERR_SCRATCH
    assert f(fake, fake, fake, fake, fake, 4, 65, 100, 100, 1, 1.0, fake, fake, None, None) == \
        SV_ERR_SHAPE
    assert f(fake, fake, fake, fake, fake, -1, 2, 100, 100, 1, 1.0, fake, fake, None, None) == \
        SV_ERR_SHAPE
    assert f(fake, fake, fake, fake, fake, 0, 2, 100, 100, 1, 1.0, fake, fake, None, None) == SV_OK
