"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments on
the host before any launch (CPU only: no call here reaches a kernel launch)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import swish_activation_backward_amd as swg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swiglu_bwd.h")

OK, NULLPTR, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3, 4
BF16, FP16, FP32 = 0, 1, 2
# fake, suitably aligned device addresses: validation must reject before touching them
P = ctypes.c_void_p(0x10000)
Q = ctypes.c_void_p(0x20000)
R = ctypes.c_void_p(0x30000)
S = ctypes.c_void_p(0x40000)
T = ctypes.c_void_p(0x50000)
U = ctypes.c_void_p(0x60000)
V = ctypes.c_void_p(0x70000)
NULL = None


@pytest.fixture(scope="module")
def lib():
    return swg.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"swiglu_bwd_b", "swiglu_bwd_w", "swiglu_bwd_x", "swish_grad"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/swiglu_bwd.h but not exported"


def test_header_is_plain_c_and_links(lib, tmp_path):
    """A C99 program (gcc -std=c99 -pedantic -Werror) includes the header, takes the address
    of every declared function, links against the in-tree library and runs its host-only
    calls: the boundary needs neither C++ nor torch."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not installed")
    names = declared_functions()
    libdir = os.path.dirname(swg.library_path())
    src = tmp_path / "main.c"
    src.write_text(
        "#include <stdio.h>\n#include \"swiglu_bwd.h\"\n"
        "static void (*const table[])(void) = {\n"
        + "".join(f"  (void (*)(void)){n},\n" for n in names)
        + "};\n"
        "int main(void) {\n"
        "  printf(\"%d\\n\", (int)(sizeof(table) / sizeof(table[0])));\n"
        "  printf(\"%s\\n\", swg_version());\n"
        "  printf(\"%zu\\n\", swiglu_bwd_b_workspace_size(220000, 1024, SWG_BF16));\n"
        "  printf(\"%d\\n\", swiglu_bwd_gemm_tile(1, 8191, 512, 1024, SWG_BF16));\n"
        "  return 0;\n}\n")
    exe = tmp_path / "main"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
           "-L", libdir, "-lswiglu_bwd", f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr[-2000:]
    lines = out.stdout.splitlines()
    assert int(lines[0]) == len(names)
    assert lines[1].startswith("swiglu_bwd ") and lines[1].endswith("gfx950")
    assert int(lines[2]) == lib.swiglu_bwd_b_workspace_size(220000, 1024, BF16)
    assert int(lines[3]) == 128   # the 128 x 128 x-stage tile at the ragged batch


def test_status_strings_and_version(lib):
    for code in range(6):
        s = lib.swg_status_string(code).decode()
        assert s.startswith(swg.STATUS[code])
    assert lib.swg_status_string(99).decode() == "unknown swg_status"
    assert swg.swg_version().startswith("swiglu_bwd")
    assert "gfx950" in swg.swg_version()
    assert lib.swg_last_hip_error() == 0


def test_time_next_call_arguments(lib):
    assert lib.swg_time_next_call(NULL, NULL) == OK      # cancels
    assert lib.swg_time_next_call(P, NULL) == INVALID
    assert lib.swg_time_next_call(NULL, Q) == INVALID
    # an argument error in the next call returns before any launch and clears the events
    assert lib.swg_time_next_call(P, Q) == OK
    assert lib.swish_grad(P, Q, R, -1, BF16, None, NULL) == INVALID
    assert lib.swish_grad(P, Q, R, 0, BF16, None, NULL) == OK


def test_swish_grad_argument_errors(lib):
    beta = ctypes.byref(ctypes.c_float(1.0))
    assert lib.swish_grad(P, Q, R, 0, BF16, beta, NULL) == OK          # empty: no work
    assert lib.swish_grad(NULL, NULL, NULL, 0, BF16, None, NULL) == OK
    assert lib.swish_grad(P, Q, R, -1, BF16, beta, NULL) == INVALID
    assert lib.swish_grad(P, Q, R, 10, 7, beta, NULL) == INVALID       # unknown dtype
    assert lib.swish_grad(NULL, Q, R, 10, BF16, beta, NULL) == NULLPTR
    assert lib.swish_grad(P, NULL, R, 10, FP16, beta, NULL) == NULLPTR
    assert lib.swish_grad(P, Q, NULL, 10, FP32, None, NULL) == NULLPTR
    odd = ctypes.c_void_p(0x10001)
    assert lib.swish_grad(odd, Q, R, 10, BF16, beta, NULL) == INVALID  # misaligned
    assert lib.swish_grad(P, Q, ctypes.c_void_p(0x10002 + 0x4), 10, FP32, beta, NULL) == INVALID
    # partial overlap of output and input is rejected; exact aliasing is allowed
    assert lib.swish_grad(P, Q, ctypes.c_void_p(0x10000 + 8), 100, BF16, beta, NULL) == INVALID
    assert lib.swish_grad(P, Q, ctypes.c_void_p(0x20000 - 8), 100, BF16, beta, NULL) == INVALID


def _i64(*v):
    return (ctypes.c_int64 * max(len(v), 1))(*v)


def test_swish_grad_strided_argument_errors(lib):
    beta = ctypes.byref(ctypes.c_float(1.0))
    f = lib.swish_grad_strided
    c2 = _i64(4, 1)
    assert f(P, Q, R, -1, _i64(4), _i64(1), _i64(1), _i64(1), BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 65, _i64(4), _i64(1), _i64(1), _i64(1), BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 2, _i64(3, 4), c2, c2, c2, 9, beta, NULL) == INVALID       # dtype
    assert f(P, Q, R, 2, NULL, c2, c2, c2, BF16, beta, NULL) == NULLPTR
    assert f(P, Q, R, 2, _i64(3, 4), NULL, c2, c2, BF16, beta, NULL) == NULLPTR
    assert f(P, Q, R, 2, _i64(3, -4), c2, c2, c2, BF16, beta, NULL) == INVALID   # negative size
    assert f(P, Q, R, 2, _i64(1 << 40, 1 << 40), c2, c2, c2, BF16, beta, NULL) == INVALID
    # empty views succeed without looking at the pointers
    assert f(NULL, NULL, NULL, 2, _i64(0, 4), c2, c2, c2, BF16, beta, NULL) == OK
    assert f(NULL, Q, R, 2, _i64(3, 4), c2, c2, c2, BF16, beta, NULL) == NULLPTR
    assert f(ctypes.c_void_p(0x10001), Q, R, 2, _i64(3, 4), c2, c2, c2, BF16, beta,
             NULL) == INVALID                                                       # misaligned
    # an output whose elements overlap: a zero stride, or strides that interleave
    assert f(P, Q, R, 2, _i64(3, 4), c2, c2, _i64(0, 1), BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 2, _i64(4, 4), c2, c2, _i64(2, 1), BF16, beta, NULL) == INVALID
    # broadcast (zero-stride) inputs are fine for validation; overlap of the output with
    # an input other than the identical view is rejected
    assert f(P, Q, ctypes.c_void_p(0x10000 + 4), 2, _i64(3, 4), c2, c2, c2, BF16, beta,
             NULL) == INVALID
    assert f(P, Q, P, 2, _i64(3, 4), _i64(1, 3), c2, c2, BF16, beta, NULL) == INVALID
    # strides whose byte span does not fit int64 (input or output), and INT64_MIN
    huge = _i64(1 << 62, 1)
    assert f(P, Q, R, 2, _i64(3, 4), huge, c2, c2, BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 2, _i64(3, 4), c2, huge, c2, BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 2, _i64(3, 4), c2, c2, huge, BF16, beta, NULL) == INVALID
    assert f(P, Q, R, 2, _i64(3, 4), _i64(-(1 << 63), 1), c2, c2, BF16, beta,
             NULL) == INVALID
    assert f(P, Q, R, 2, _i64(1, 4), c2, c2, _i64(-(1 << 63), 1), BF16, beta,
             NULL) == INVALID
    # nine dimensions that cannot be merged (x runs the other way round)
    sizes = _i64(*([2] * 9))
    rowmajor = _i64(*[1 << (8 - d) for d in range(9)])
    colmajor = _i64(*[1 << d for d in range(9)])
    assert f(P, Q, R, 9, sizes, rowmajor, colmajor, rowmajor, BF16, beta, NULL) == UNSUPPORTED


def test_b_stage_argument_errors(lib):
    ws = swg.swiglu_bwd_b_workspace_size
    import torch
    M, N = 1000, 64
    need = ws(M, N, torch.bfloat16)
    assert need > 0
    args = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                         (("dy", P), ("g", Q), ("fc", R), ("dg", S), ("dfc", T), ("dbg", U),
                          ("dbfc", V), ("M", M), ("N", N), ("dt", BF16), ("w", P),
                          ("wb", need), ("s", NULL))]
    assert lib.swiglu_bwd_b(*args(M=0)) == OK
    assert lib.swiglu_bwd_b(*args(N=0)) == OK
    assert lib.swiglu_bwd_b(*args(M=0, dy=NULL, w=NULL, wb=0)) == OK
    assert lib.swiglu_bwd_b(*args(M=-1)) == INVALID
    assert lib.swiglu_bwd_b(*args(N=-5)) == INVALID
    assert lib.swiglu_bwd_b(*args(dt=3)) == INVALID
    for k in ("dy", "g", "fc", "dg", "dfc", "dbg", "dbfc"):
        assert lib.swiglu_bwd_b(*args(**{k: NULL})) == NULLPTR, k
    assert lib.swiglu_bwd_b(*args(wb=need - 1)) == WORKSPACE
    assert lib.swiglu_bwd_b(*args(w=NULL)) == NULLPTR
    assert lib.swiglu_bwd_b(*args(dbg=ctypes.c_void_p(0x60001))) == INVALID


def test_gemm_argument_errors(lib):
    import torch
    M, K, N = 4096, 64, 128
    need = swg.swiglu_bwd_w_workspace_size(M, K, N, torch.bfloat16)
    wa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("x", P), ("dg", Q), ("dfc", R), ("dwg", S), ("dwfc", T), ("M", M),
                        ("K", K), ("N", N), ("dt", BF16), ("w", U), ("wb", need), ("s", NULL))]
    assert lib.swiglu_bwd_w(*wa(M=0)) == OK
    assert lib.swiglu_bwd_w(*wa(K=0)) == OK
    assert lib.swiglu_bwd_w(*wa(M=-1)) == INVALID
    assert lib.swiglu_bwd_w(*wa(dt=9)) == INVALID
    assert lib.swiglu_bwd_w(*wa(K=60)) == UNSUPPORTED                 # 16-bit: multiples of 8
    assert lib.swiglu_bwd_w(*wa(N=100)) == UNSUPPORTED
    assert lib.swiglu_bwd_w(*wa(dt=FP32, K=62)) == UNSUPPORTED        # fp32: multiples of 4
    assert lib.swiglu_bwd_w(*wa(dt=FP32, N=102)) == UNSUPPORTED
    assert lib.swiglu_bwd_w(*wa(dt=FP32, x=NULL)) == NULLPTR          # fp32 is a valid dtype
    for k in ("x", "dg", "dfc", "dwg", "dwfc"):
        assert lib.swiglu_bwd_w(*wa(**{k: NULL})) == NULLPTR, k
    if need > 0:
        assert lib.swiglu_bwd_w(*wa(wb=need - 1)) == WORKSPACE
        assert lib.swiglu_bwd_w(*wa(w=NULL)) == NULLPTR
    xa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("dg", P), ("dfc", Q), ("wg", R), ("wfc", S), ("dx", T), ("M", M),
                        ("K", K), ("N", N), ("dt", BF16), ("s", NULL))]
    assert lib.swiglu_bwd_x(*xa(M=0)) == OK
    assert lib.swiglu_bwd_x(*xa(K=0, dx=NULL)) == OK
    assert lib.swiglu_bwd_x(*xa(K=-8)) == INVALID
    assert lib.swiglu_bwd_x(*xa(N=12)) == UNSUPPORTED
    assert lib.swiglu_bwd_x(*xa(dt=FP32, N=10)) == UNSUPPORTED
    assert lib.swiglu_bwd_x(*xa(dt=FP32, dg=NULL)) == NULLPTR
    for k in ("dg", "dfc", "wg", "wfc", "dx"):
        assert lib.swiglu_bwd_x(*xa(**{k: NULL})) == NULLPTR, k
    assert lib.swiglu_bwd_x(*xa(N=0, dx=NULL)) == NULLPTR
    assert lib.swiglu_bwd_x(*xa(dg=ctypes.c_void_p(0x10008))) == UNSUPPORTED


def test_fused_wx_argument_errors(lib):
    import torch
    M, K, N = 4096, 64, 128
    need = swg.swiglu_bwd_wx_workspace_size(M, K, N, torch.bfloat16)
    assert need == swg.swiglu_bwd_wx_workspace_size(M, K, N, torch.float16)
    need32 = swg.swiglu_bwd_wx_workspace_size(M, K, N, torch.float32)
    assert need32 == swg.swiglu_bwd_w_workspace_size(M, K, N, torch.float32) > 0
    W_ = ctypes.c_void_p(0x80000)
    fa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("x", P), ("dg", Q), ("dfc", R), ("wg", S), ("wfc", T), ("dwg", U),
                        ("dwfc", V), ("dx", W_), ("M", M), ("K", K), ("N", N), ("dt", BF16),
                        ("w", ctypes.c_void_p(0x100000)), ("wb", need), ("s", NULL))]
    f = lib.swiglu_bwd_wx
    assert f(*fa(M=0)) == OK
    assert f(*fa(K=0, dx=NULL)) == OK
    assert f(*fa(M=-1)) == INVALID
    assert f(*fa(dt=9)) == INVALID
    assert f(*fa(dt=FP32, K=66)) == UNSUPPORTED      # fp32: K, N multiples of 4
    assert f(*fa(dt=FP32, wb=need32 - 1)) == WORKSPACE   # fp32 runs w then x
    assert f(*fa(K=60)) == UNSUPPORTED
    assert f(*fa(N=100)) == UNSUPPORTED
    for k in ("x", "dg", "dfc", "wg", "wfc", "dwg", "dwfc", "dx"):
        assert f(*fa(**{k: NULL})) == NULLPTR, k
    assert f(*fa(N=0, dx=NULL)) == NULLPTR
    assert f(*fa(dx=ctypes.c_void_p(0x80008))) == UNSUPPORTED
    assert f(*fa(dwg=ctypes.c_void_p(0x60004))) == UNSUPPORTED
    if need > 0:
        assert f(*fa(wb=need - 1)) == WORKSPACE
        assert f(*fa(w=NULL)) == NULLPTR
    # overlaps (a small shape, so the fake buffers are otherwise disjoint)
    sm = lambda **kw: fa(M=4, K=8, N=8, w=NULL, wb=0, **kw)  # noqa: E731
    for k, alias in (("dx", P), ("dwg", Q), ("dwfc", U), ("dx", ctypes.c_void_p(0x50040))):
        assert f(*sm(**{k: alias})) == INVALID, (k, alias)


def test_forward_argument_errors(lib):
    M, K, N = 4096, 64, 128
    W_ = ctypes.c_void_p(0x80000)
    fa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("x", P), ("wg", Q), ("wfc", R), ("bg", S), ("bfc", T), ("g", U),
                        ("fc", V), ("y", W_), ("M", M), ("K", K), ("N", N), ("dt", BF16),
                        ("s", NULL))]
    assert lib.swiglu_fwd(*fa(M=0)) == OK
    assert lib.swiglu_fwd(*fa(N=0)) == OK
    assert lib.swiglu_fwd(*fa(M=-1)) == INVALID
    assert lib.swiglu_fwd(*fa(dt=FP32, K=36, g=NULL)) == NULLPTR   # fp32 accepted
    assert lib.swiglu_fwd(*fa(dt=FP32, N=10)) == UNSUPPORTED        # K, N multiples of 4
    assert lib.swiglu_fwd(*fa(dt=FP32, bg=ctypes.c_void_p(0x40002))) == INVALID
    assert lib.swiglu_fwd(*fa(dt=7)) == INVALID
    assert lib.swiglu_fwd(*fa(K=60)) == UNSUPPORTED
    assert lib.swiglu_fwd(*fa(N=100)) == UNSUPPORTED
    for k in ("x", "wg", "wfc", "g", "fc", "y"):
        assert lib.swiglu_fwd(*fa(**{k: NULL})) == NULLPTR, k
    assert lib.swiglu_fwd(*fa(x=ctypes.c_void_p(0x10008))) == UNSUPPORTED
    assert lib.swiglu_fwd(*fa(bg=ctypes.c_void_p(0x40001))) == INVALID


def test_noalloc_b_stage_argument_errors(lib):
    """The static-scratch b stage validates like swiglu_bwd_b, and refuses shapes whose
    partials exceed its array (before any launch)."""
    import torch
    M, N = 1000, 64
    args = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                         (("dy", P), ("g", Q), ("fc", R), ("dg", S), ("dfc", T), ("dbg", U),
                          ("dbfc", V), ("M", M), ("N", N), ("dt", BF16), ("s", NULL))]
    f = lib.swiglu_bwd_b_noalloc
    assert f(*args(M=0)) == OK
    assert f(*args(N=0, dy=NULL)) == OK
    assert f(*args(M=-1)) == INVALID
    assert f(*args(dt=3)) == INVALID
    for k in ("dy", "g", "fc", "dg", "dfc", "dbg", "dbfc"):
        assert f(*args(**{k: NULL})) == NULLPTR, k
    assert f(*args(dbg=ctypes.c_void_p(0x60001))) == INVALID
    assert f(*args(M=4, N=8, dg=P)) == INVALID                         # output overlaps dy
    # partials beyond the 16 MiB array: N = 2^22 bf16 columns need one walker's 2N floats
    big_n = 1 << 22
    assert swg.swiglu_bwd_b_workspace_size(8192, 1 << 21, torch.bfloat16) <= 16 << 20
    assert swg.swiglu_bwd_b_workspace_size(8192, big_n, torch.bfloat16) > 16 << 20
    assert f(*args(M=8192, N=big_n)) == WORKSPACE
    assert swg.swiglu_bwd_b_workspace_size(220000, 1024, torch.bfloat16) <= 16 << 20
    assert swg.swiglu_bwd_b_workspace_size(16384, 14336, torch.bfloat16) <= 16 << 20


def test_overlapping_outputs_are_rejected(lib):
    """An output that overlaps another buffer is refused on the host (each call below is
    otherwise valid, so only the overlap rule can reject it: none reaches a launch)."""
    M, K, N = 4, 8, 8                      # 64-byte [M, N] tensors, fake buffers 64 KiB apart
    ba = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("dy", P), ("g", Q), ("fc", R), ("dg", S), ("dfc", T), ("dbg", U),
                        ("dbfc", V), ("M", M), ("N", N), ("dt", BF16),
                        ("w", ctypes.c_void_p(0x90000)), ("wb", 1 << 20), ("s", NULL))]
    for k, alias in (("dg", P), ("dfc", Q), ("dg", ctypes.c_void_p(0x10010)), ("dbg", S),
                     ("dbfc", ctypes.c_void_p(0x50008)), ("dfc", S), ("w", T), ("w", P)):
        assert lib.swiglu_bwd_b(*ba(**{k: alias})) == INVALID, (k, alias)
    wa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("x", P), ("dg", Q), ("dfc", R), ("dwg", S), ("dwfc", T), ("M", M),
                        ("K", K), ("N", N), ("dt", BF16), ("w", U), ("wb", 1 << 20),
                        ("s", NULL))]
    for k, alias in (("dwg", P), ("dwfc", R), ("dwfc", S), ("dwg", ctypes.c_void_p(0x20010))):
        assert lib.swiglu_bwd_w(*wa(**{k: alias})) == INVALID, (k, alias)
    # a split over M (4096 rows, 2 x 1 tiles): the workspace is used and may not overlap dw
    import torch
    need = swg.swiglu_bwd_w_workspace_size(4096, K, N, torch.bfloat16)
    assert need > 0
    assert lib.swiglu_bwd_w(*wa(M=4096, w=S, wb=need)) == INVALID
    xa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("dg", P), ("dfc", Q), ("wg", R), ("wfc", S), ("dx", T), ("M", M),
                        ("K", K), ("N", N), ("dt", BF16), ("s", NULL))]
    for alias in (P, Q, R, S, ctypes.c_void_p(0x40030)):
        assert lib.swiglu_bwd_x(*xa(dx=alias)) == INVALID, alias
    W_ = ctypes.c_void_p(0x80000)
    fa = lambda **kw: [kw.get(k, d) for k, d in  # noqa: E731
                       (("x", P), ("wg", Q), ("wfc", R), ("bg", S), ("bfc", T), ("g", U),
                        ("fc", V), ("y", W_), ("M", M), ("K", K), ("N", N), ("dt", BF16),
                        ("s", NULL))]
    for k, alias in (("g", P), ("fc", U), ("y", V), ("y", S), ("g", ctypes.c_void_p(0x50000)),
                     ("fc", ctypes.c_void_p(0x20020))):
        assert lib.swiglu_fwd(*fa(**{k: alias})) == INVALID, (k, alias)


def test_gemm_tile_query_and_override(lib):
    """The planner's tile choice (host arithmetic, no device needed) and the thread-local
    override that the GPU tests use to run every GEMM shape at both tile sizes."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    t = swg.swiglu_bwd_gemm_tile
    # the large-batch and LLM-sized FFNs keep 256 x 256 tiles in the x stage; the tiny and
    # ragged batches, which have too few of them for 256 CUs, take 128 x 128
    assert t("x", 220000, 512, 1024, bf) == 256 and t("x", 16384, 4096, 14336, bf) == 256
    assert t("x", 8191, 512, 1024, bf) == 128 and t("x", 256, 64, 128, bf) == 128
    assert t("w", 16384, 4096, 14336, bf) == 256 and t("w", 8191, 512, 1024, bf) == 128
    assert t("wx", 220000, 512, 1024, bf) == 256 and t("wx", 8191, 512, 1024, bf) == 128
    for st in ("w", "x", "wx"):
        assert t(st, 0, 64, 128, bf) == 0 and t(st, 256, 64, 128, f32) == 0
        assert t(st, 256, 60, 128, bf) == 0          # K not a multiple of 8
    assert lib.swiglu_bwd_gemm_tile(7, 256, 64, 128, BF16) == 0
    for bad in (64, -1, 512, 1):
        assert lib.swg_set_gemm_tile(bad) == INVALID
    try:
        for edge in (128, 256):
            assert lib.swg_set_gemm_tile(edge) == OK
            for st in ("w", "x", "wx"):
                assert t(st, 220000, 512, 1024, bf) == edge
                assert t(st, 8191, 512, 1024, bf) == edge
            # w stage at M = 8191: the M splits fill one round of 256 workgroups with the
            # tiles of that size, at least 512 rows each
            tiles = (512 // edge) * 2 * (1024 // edge)
            splits = swg.swiglu_bwd_w_workspace_size(8191, 512, 1024, bf) // (512 * 2048 * 4)
            assert splits == min(256 // tiles, 8191 // 512)
    finally:
        assert lib.swg_set_gemm_tile(0) == OK
    assert t("x", 8191, 512, 1024, bf) == 128 and t("x", 220000, 512, 1024, bf) == 256


def test_fused_plan_runs_large_unsplit_shapes_as_two_stages():
    """Where the dW grid needs no M split and each stage fills the GPU alone, swiglu_bwd_wx
    runs the w stage and then the x stage: its workspace is the w stage's, and the tile it
    reports is the x stage's."""
    import torch
    bf = torch.bfloat16
    wx, w = swg.swiglu_bwd_wx_workspace_size, swg.swiglu_bwd_w_workspace_size
    t = swg.swiglu_bwd_gemm_tile
    for (M, K, N) in ((16384, 4096, 14336), (4096, 4096, 14336), (4096, 4096, 4096)):
        assert wx(M, K, N, bf) == w(M, K, N, bf) == 0
        assert t("wx", M, K, N, bf) == t("x", M, K, N, bf)
    # fused where the M split shares rows (large batch) or one stage alone under-fills
    per_split = 512 * 2048 * 4
    assert wx(220000, 512, 1024, bf) == 8 * per_split      # 8 splits x 16 dW tiles
    assert wx(2048, 4096, 4096, bf) == 0 and t("wx", 2048, 4096, 4096, bf) == 256


def test_gemm_plan_invariants_over_random_shapes():
    """Over seeded shapes (through the public queries only): the tile is 128 or 256; the
    w stage's M splits (workspace / (K * 2N * 4 bytes)) keep tiles x splits within one
    round of 256 workgroups, leave every split at least 512 rows and appear only when
    the tile grid is short of 256; the fused pass's workspace is its splits' or, when it
    runs the two stages, the w stage's; every query agrees between two calls."""
    import numpy as np
    import torch
    bf = torch.bfloat16
    rng = np.random.default_rng(77)
    for _ in range(400):
        M = int(rng.integers(1, 300000))
        K = int(rng.integers(1, 600)) * 8
        N = int(rng.integers(1, 2000)) * 8
        per_split = K * 2 * N * 4
        for stage in ("w", "x", "wx"):
            e = swg.swiglu_bwd_gemm_tile(stage, M, K, N, bf)
            assert e in (128, 256), (stage, M, K, N, e)
        e = swg.swiglu_bwd_gemm_tile("w", M, K, N, bf)
        tiles = -(-K // e) * 2 * -(-N // e)
        ws = swg.swiglu_bwd_w_workspace_size(M, K, N, bf)
        assert ws % per_split == 0
        splits = ws // per_split
        if splits:
            assert splits >= 2 and tiles * splits <= 256 and tiles < 256, (M, K, N, splits)
            assert M // splits >= 512 - 32, (M, K, N, splits)   # rows per split, 32-rounded
        wx = swg.swiglu_bwd_wx_workspace_size(M, K, N, bf)
        assert wx % per_split == 0 and wx // per_split <= 256
        assert wx == swg.swiglu_bwd_wx_workspace_size(M, K, N, bf)
        assert ws == swg.swiglu_bwd_w_workspace_size(M, K, N, bf)


def test_workspace_queries():
    import torch
    b = swg.swiglu_bwd_b_workspace_size
    w = swg.swiglu_bwd_w_workspace_size
    assert b(0, 128, torch.bfloat16) == 0 and b(128, 0, torch.bfloat16) == 0
    assert w(0, 64, 128, torch.bfloat16) == 0
    assert w(100, 64, 128, torch.float32) == 0            # unsupported -> 0
    # b: one fp32 partial row [2N] per row chunk, a bounded number of chunks
    for (M, N) in ((256, 128), (8191, 1024), (220000, 1024), (16384, 14336), (1, 8), (37, 13)):
        nb = b(M, N, torch.bfloat16)
        assert nb % (2 * N * 4) == 0 and 0 < nb // (2 * N * 4) <= max(M, 1)
        assert nb // (2 * N * 4) <= 4096
    # b plan: strips of at most 32 16-byte vector columns; units of whole 8-row passes and
    # a power-of-two walker count per strip (or every unit) chosen for whole rounds of 256
    # resident workgroups, except for small batches (at most 4096 workgroups that way),
    # which take units of one 4-row pass and one walker per unit; pinned at the workload
    # shapes
    for (M, N, dt, strips, walkers) in ((220000, 1024, torch.bfloat16, 4, 256),
                                        (16384, 14336, torch.bfloat16, 56, 32),
                                        (16384, 14336, torch.float32, 112, 16),
                                        (220000, 1024, torch.float32, 8, 128),
                                        (8191, 1024, torch.float16, 4, 256),
                                        (256, 128, torch.bfloat16, 1, 4),
                                        (4097, 24, torch.bfloat16, 1, 17),
                                        (65536, 1024, torch.bfloat16, 4, 1024)):
        vec = 4 if dt == torch.float32 else 8
        cv = N // vec if N % vec == 0 else N          # 16-byte vector columns
        tx = 1
        while tx < 32 and tx < cv:
            tx *= 2
        assert -(-cv // tx) == strips
        got = b(M, N, dt) // (2 * N * 4)
        assert got == walkers, (M, N, dt, got)
        unit = max(64, 8 * (256 // tx))               # rows per unit: whole 8-row passes
        nunits = -(-M // unit)
        if strips * nunits <= 4096:                   # small batch: one 4-row pass per unit
            assert got == min(-(-M // (4 * (256 // tx))), 4096 // strips)
            continue
        assert got == nunits or (got & (got - 1)) == 0    # a power of two, or every unit
        assert strips * got >= 1024 or got == nunits
        assert strips * got < 8 * max(1024, strips)
    # w: the split-M partials only when the output tile grid is small
    assert w(16384, 4096, 14336, torch.bfloat16) == 0
    s3 = w(220000, 512, 1024, torch.bfloat16)
    assert s3 % (512 * 2048 * 4) == 0 and 2 <= s3 // (512 * 2048 * 4) <= 256
    assert w(256, 64, 128, torch.bfloat16) == 0


def test_binding_checks_shapes_without_gpu():
    import torch
    x = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        swg.swish_grad(x, torch.zeros(4, 9, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        swg.swiglu_bwd_x(x, x, torch.zeros(8, 8, dtype=torch.float16), x, x)
    # well-formed host tensors are refused before any library call
    with pytest.raises(ValueError, match="GPU only"):
        swg.swish_grad(x, x)
    with pytest.raises(ValueError, match="GPU only"):
        swg.swish_grad(x.t(), x.t())        # non-contiguous: the strided entry point
    w = torch.zeros(8, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU only"):
        swg.swiglu_fwd(x, w, w, None, None, x.clone(), x.clone(), x.clone())


def test_product_path_has_no_cpu_fallback():
    """The package must not import the oracle or any CPU implementation."""
    pkg = os.path.join(ROOT, "swish_activation_backward_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("the oracle", ""), f
                assert "numpy" not in text, f


def test_binding_checks_every_operand_layout():
    """Each operand's layout is checked, also the ones whose shape defines the sizes (x
    of the forward, dg of the x stage): a transposed view is refused, not read as if it
    were row-major."""
    import torch
    xt = torch.zeros(8, 4, dtype=torch.bfloat16).t()          # [4, 8], not contiguous
    w = torch.zeros(8, 8, dtype=torch.bfloat16)
    o = torch.zeros(4, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="contiguous"):
        swg.swiglu_fwd(xt, w, w, None, None, o, o.clone(), o.clone())
    with pytest.raises(ValueError, match="contiguous"):
        swg.swiglu_bwd_x(xt, o, w, w, torch.zeros(4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="dtype"):
        swg.swiglu_fwd(o.half(), w, w, None, None, o, o.clone(), o.clone())
