"""ctypes binding of libswiglu_bwd.so: argument marshalling only.

Each function has the name of the C entry point it calls and takes torch CUDA (HIP)
tensors: it checks shapes and dtypes, turns tensors into device pointers and sizes,
passes torch's current stream, and raises ``SwgError`` on a non-zero status.  All
arithmetic happens in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = ["SwgError", "load_library", "library_path", "swish_grad", "swish_grad_strided",
           "swiglu_bwd_b", "swiglu_bwd_b_noalloc", "swiglu_bwd_w", "swiglu_bwd_x", "swiglu_fwd",
           "swiglu_bwd_b_workspace_size", "swiglu_bwd_w_workspace_size", "swg_version",
           "swg_time_next_call", "swiglu_bwd_wx", "swiglu_bwd_wx_workspace_size",
           "swiglu_bwd_gemm_tile", "swg_set_gemm_tile", "DTYPE_CODE", "STATUS"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libswiglu_bwd.so"

DTYPE_CODE = {torch.bfloat16: 0, torch.float16: 1, torch.float32: 2}
STATUS = {0: "SWG_OK", 1: "SWG_ERR_NULLPTR", 2: "SWG_ERR_INVALID", 3: "SWG_ERR_UNSUPPORTED",
          4: "SWG_ERR_WORKSPACE", 5: "SWG_ERR_HIP"}

_lock = threading.Lock()
_lib = None


class SwgError(RuntimeError):
    def __init__(self, call: str, status: int, lib):
        self.status = status
        msg = lib.swg_status_string(status).decode()
        if status == 5:
            msg += f" (hipError_t {lib.swg_last_hip_error()})"
        super().__init__(f"{call}: {msg}")


def library_path() -> str:
    return os.environ.get("SWIGLU_BWD_LIB", os.path.join(_HERE, _LIB_NAME))


def load_library():
    """Load the HIP library (raises if it has not been built: no fallback exists)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m swish_activation_backward_amd.build`"
                " (the SwiGLU backward has no CPU fallback)")
        lib = ctypes.CDLL(path)
        vp, i64, sz, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
        lib.swish_grad.argtypes = [vp, vp, vp, i64, i32, ctypes.POINTER(ctypes.c_float), vp]
        lib.swish_grad.restype = i32
        pi64 = ctypes.POINTER(ctypes.c_int64)
        lib.swish_grad_strided.argtypes = [vp, vp, vp, i32, pi64, pi64, pi64, pi64, i32,
                                           ctypes.POINTER(ctypes.c_float), vp]
        lib.swish_grad_strided.restype = i32
        lib.swiglu_bwd_b.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp, sz, vp]
        lib.swiglu_bwd_b.restype = i32
        lib.swiglu_bwd_b_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i32, vp]
        lib.swiglu_bwd_b_noalloc.restype = i32
        lib.swiglu_bwd_b_workspace_size.argtypes = [i64, i64, i32]
        lib.swiglu_bwd_b_workspace_size.restype = sz
        lib.swiglu_bwd_w.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp, sz, vp]
        lib.swiglu_bwd_w.restype = i32
        lib.swiglu_bwd_w_workspace_size.argtypes = [i64, i64, i64, i32]
        lib.swiglu_bwd_w_workspace_size.restype = sz
        lib.swiglu_bwd_x.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
        lib.swiglu_bwd_x.restype = i32
        lib.swiglu_bwd_wx.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp,
                                      sz, vp]
        lib.swiglu_bwd_wx.restype = i32
        lib.swiglu_bwd_wx_workspace_size.argtypes = [i64, i64, i64, i32]
        lib.swiglu_bwd_wx_workspace_size.restype = sz
        lib.swiglu_bwd_gemm_tile.argtypes = [i32, i64, i64, i64, i32]
        lib.swiglu_bwd_gemm_tile.restype = i32
        lib.swg_set_gemm_tile.argtypes = [i32]
        lib.swg_set_gemm_tile.restype = i32
        lib.swiglu_fwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i32, vp]
        lib.swiglu_fwd.restype = i32
        lib.swg_status_string.argtypes = [i32]
        lib.swg_status_string.restype = ctypes.c_char_p
        lib.swg_last_hip_error.argtypes = []
        lib.swg_last_hip_error.restype = i32
        lib.swg_time_next_call.argtypes = [vp, vp]
        lib.swg_time_next_call.restype = i32
        lib.swg_version.argtypes = []
        lib.swg_version.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _ptr(t):
    """Device pointer of a GPU tensor; host tensors are refused (the kernels would
    dereference host addresses)."""
    if t is None:
        return None
    if t.device.type != "cuda":
        raise ValueError(f"tensor on {t.device}: the library computes on the GPU only "
                         f"(move inputs and outputs to a cuda device)")
    return ctypes.c_void_p(t.data_ptr())


def _on_device(device):
    """Context that makes ``device`` HIP's current device for the launch (the library
    launches on the current device); host tensors are refused."""
    if device.type != "cuda":
        raise ValueError(f"tensor on {device}: the library computes on the GPU only "
                         f"(move inputs and outputs to a cuda device)")
    return torch.cuda.device(device)


def _stream(stream, device):
    """The stream handle to launch on: ``stream``, else torch's current stream of the
    tensors' device."""
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(call, status, lib):
    if status != 0:
        raise SwgError(call, status, lib)


def _dense(name, t, dtype, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _dtype_code(t):
    if t.dtype not in DTYPE_CODE:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPE_CODE[t.dtype]


def _workspace(nbytes, workspace, device, stream):
    """The caller's workspace (checked), or a new one from torch's allocator.  A new one is
    marked as used on ``stream`` so that the allocator does not hand its memory out again
    before the kernels queued there have finished with it."""
    if nbytes == 0:
        return workspace
    if workspace is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        if stream is not None:
            ws.record_stream(stream)
        return ws
    if workspace.numel() * workspace.element_size() < nbytes or not workspace.is_contiguous():
        raise ValueError(f"workspace needs {nbytes} contiguous bytes")
    if workspace.device != device:
        raise ValueError(f"workspace is on {workspace.device}, expected {device}")
    return workspace


def swg_version() -> str:
    return load_library().swg_version().decode()


def swg_time_next_call(start, stop):
    """Attach two ``torch.cuda.Event`` (timing enabled, each recorded at least once so that
    torch has created it) to the kernels of the next library call on this thread: after it,
    ``start.elapsed_time(stop)`` is the span from its first kernel's start to its last
    kernel's end.  ``None, None`` cancels."""
    lib = load_library()
    handles = []
    for name, e in (("start", start), ("stop", stop)):
        if e is None:
            handles.append(None)
            continue
        h = e.cuda_event
        if not h:
            raise ValueError(f"{name} event has no HIP event yet: record it once first")
        handles.append(ctypes.c_void_p(h))
    _check("swg_time_next_call", lib.swg_time_next_call(*handles), lib)


def _same_kind(name, t, dtype, shape, device):
    """dtype, shape and device checks without a layout requirement (strided calls)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def swish_grad(grad, x, grad_x=None, beta=None, stream=None):
    """grad_x = grad * sigma(beta x) * (1 + beta x (1 - sigma(beta x)))  (elementwise, any
    shape).  ``beta`` None means 1.0; ``grad_x`` may be ``grad`` or ``x`` (in place).
    Contiguous tensors go to ``swish_grad``; any other layout (transposed, sliced,
    broadcast inputs, a non-contiguous output) to ``swish_grad_strided``."""
    _same_kind("x", x, grad.dtype, grad.shape, grad.device)
    if grad_x is None:
        grad_x = torch.empty(grad.shape, dtype=grad.dtype, device=grad.device)
    _same_kind("grad_x", grad_x, grad.dtype, grad.shape, grad.device)
    if not (grad.is_contiguous() and x.is_contiguous() and grad_x.is_contiguous()):
        return swish_grad_strided(grad, x, grad_x, beta=beta, stream=stream)
    lib = load_library()
    b = None if beta is None else ctypes.byref(ctypes.c_float(beta))
    with _on_device(grad.device):
        st = lib.swish_grad(_ptr(grad), _ptr(x), _ptr(grad_x), grad.numel(), _dtype_code(grad),
                            b, _stream(stream, grad.device))
    _check("swish_grad", st, lib)
    return grad_x


def swish_grad_strided(grad, x, grad_x, beta=None, stream=None):
    """The Swish gradient over tensors of one shape with any strides (the C entry point
    of the same name: passes torch's sizes and element strides)."""
    _same_kind("x", x, grad.dtype, grad.shape, grad.device)
    _same_kind("grad_x", grad_x, grad.dtype, grad.shape, grad.device)
    lib = load_library()
    nd = grad.dim()
    arr = ctypes.c_int64 * max(nd, 1)
    sizes = arr(*grad.shape)
    sg, sx, so = arr(*grad.stride()), arr(*x.stride()), arr(*grad_x.stride())
    b = None if beta is None else ctypes.byref(ctypes.c_float(beta))
    with _on_device(grad.device):
        st = lib.swish_grad_strided(_ptr(grad), _ptr(x), _ptr(grad_x), nd, sizes, sg, sx, so,
                                    _dtype_code(grad), b, _stream(stream, grad.device))
    _check("swish_grad_strided", st, lib)
    return grad_x


def swiglu_bwd_b_workspace_size(M: int, N: int, dtype) -> int:
    return int(load_library().swiglu_bwd_b_workspace_size(M, N, DTYPE_CODE[dtype]))


def swiglu_bwd_w_workspace_size(M: int, K: int, N: int, dtype) -> int:
    return int(load_library().swiglu_bwd_w_workspace_size(M, K, N, DTYPE_CODE[dtype]))


def swiglu_bwd_b(dy, g, fc, dg, dfc, db_g, db_fc, workspace=None, stream=None):
    """b stage: writes dg, dfc [M, N]; accumulates db_g, db_fc [N] (+=)."""
    lib = load_library()
    if dy.dim() != 2:
        raise ValueError("dy must be [M, N]")
    M, N = dy.shape
    dt, dev = dy.dtype, dy.device
    for name, t in (("dy", dy), ("g", g), ("fc", fc), ("dg", dg), ("dfc", dfc)):
        _dense(name, t, dt, (M, N), dev)
    for name, t in (("db_g", db_g), ("db_fc", db_fc)):
        if t.numel() != N:
            raise ValueError(f"{name} must hold N = {N} elements")
        _dense(name, t, dt, t.shape, dev)
    code = _dtype_code(dy)
    nbytes = int(lib.swiglu_bwd_b_workspace_size(M, N, code))
    with _on_device(dev):
        ws = _workspace(nbytes, workspace, dev, stream)
        st = lib.swiglu_bwd_b(_ptr(dy), _ptr(g), _ptr(fc), _ptr(dg), _ptr(dfc), _ptr(db_g),
                              _ptr(db_fc), M, N, code, _ptr(ws), 0 if ws is None else
                              ws.numel() * ws.element_size(), _stream(stream, dev))
    _check("swiglu_bwd_b", st, lib)


def swiglu_bwd_b_noalloc(dy, g, fc, dg, dfc, db_g, db_fc, stream=None):
    """b stage with the column partials in the library's static device array (no
    workspace, no allocation); same results as ``swiglu_bwd_b``."""
    lib = load_library()
    if dy.dim() != 2:
        raise ValueError("dy must be [M, N]")
    M, N = dy.shape
    dt, dev = dy.dtype, dy.device
    for name, t in (("dy", dy), ("g", g), ("fc", fc), ("dg", dg), ("dfc", dfc)):
        _dense(name, t, dt, (M, N), dev)
    for name, t in (("db_g", db_g), ("db_fc", db_fc)):
        if t.numel() != N:
            raise ValueError(f"{name} must hold N = {N} elements")
        _dense(name, t, dt, t.shape, dev)
    with _on_device(dev):
        st = lib.swiglu_bwd_b_noalloc(_ptr(dy), _ptr(g), _ptr(fc), _ptr(dg), _ptr(dfc),
                                      _ptr(db_g), _ptr(db_fc), M, N, _dtype_code(dy),
                                      _stream(stream, dev))
    _check("swiglu_bwd_b_noalloc", st, lib)


def swiglu_bwd_w(x, dg, dfc, dw_g, dw_fc, workspace=None, stream=None):
    """w stage: [dw_g | dw_fc] (each [K, N]) += x^T [dg | dfc]."""
    lib = load_library()
    if x.dim() != 2 or dg.dim() != 2:
        raise ValueError("x must be [M, K] and dg [M, N]")
    M, K = x.shape
    N = dg.shape[1]
    dt, dev = x.dtype, x.device
    _dense("x", x, dt, (M, K), dev)
    for name, t in (("dg", dg), ("dfc", dfc)):
        _dense(name, t, dt, (M, N), dev)
    for name, t in (("dw_g", dw_g), ("dw_fc", dw_fc)):
        _dense(name, t, dt, (K, N), dev)
    code = _dtype_code(x)
    nbytes = int(lib.swiglu_bwd_w_workspace_size(M, K, N, code))
    with _on_device(dev):
        ws = _workspace(nbytes, workspace, dev, stream)
        st = lib.swiglu_bwd_w(_ptr(x), _ptr(dg), _ptr(dfc), _ptr(dw_g), _ptr(dw_fc), M, K, N,
                              code, _ptr(ws), 0 if ws is None else ws.numel() * ws.element_size(),
                              _stream(stream, dev))
    _check("swiglu_bwd_w", st, lib)


def swiglu_bwd_x(dg, dfc, w_g, w_fc, dx, stream=None):
    """x stage: dx [M, K] = dg W_g^T + dfc W_fc^T (overwritten)."""
    lib = load_library()
    if dg.dim() != 2 or w_g.dim() != 2:
        raise ValueError("dg must be [M, N] and w_g [K, N]")
    M, N = dg.shape
    K = w_g.shape[0]
    dt, dev = dg.dtype, dg.device
    for name, t in (("dg", dg), ("dfc", dfc)):
        _dense(name, t, dt, (M, N), dev)
    for name, t in (("w_g", w_g), ("w_fc", w_fc)):
        _dense(name, t, dt, (K, N), dev)
    _dense("dx", dx, dt, (M, K), dev)
    with _on_device(dev):
        st = lib.swiglu_bwd_x(_ptr(dg), _ptr(dfc), _ptr(w_g), _ptr(w_fc), _ptr(dx), M, K, N,
                              _dtype_code(dg), _stream(stream, dev))
    _check("swiglu_bwd_x", st, lib)


def swiglu_bwd_wx_workspace_size(M: int, K: int, N: int, dtype) -> int:
    return int(load_library().swiglu_bwd_wx_workspace_size(M, K, N, DTYPE_CODE[dtype]))


_GEMM_STAGE = {"w": 0, "x": 1, "wx": 2}


def swiglu_bwd_gemm_tile(stage: str, M: int, K: int, N: int, dtype) -> int:
    """Output tile edge (256 or 128) the planner picks for stage "w", "x" or "wx" (the fused
    pass) at this shape; 0 where the stage does not use the bf16 / fp16 tiles."""
    return int(load_library().swiglu_bwd_gemm_tile(_GEMM_STAGE[stage], M, K, N,
                                                   DTYPE_CODE[dtype]))


def swg_set_gemm_tile(edge: int) -> None:
    """Make the GEMM calls (and workspace queries) on this thread use tile edge 256 or 128
    instead of the planner's choice; 0 restores the planner."""
    lib = load_library()
    _check("swg_set_gemm_tile", lib.swg_set_gemm_tile(int(edge)), lib)


def swiglu_bwd_wx(x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx, workspace=None, stream=None):
    """Fused w + x pass: [dw_g | dw_fc] += x^T [dg | dfc] and dx = [dg | dfc] [W_g | W_fc]^T
    (overwritten) in one launch over [dg | dfc]."""
    lib = load_library()
    if x.dim() != 2 or dg.dim() != 2 or w_g.dim() != 2:
        raise ValueError("x must be [M, K], dg [M, N] and w_g [K, N]")
    M, K = x.shape
    N = dg.shape[1]
    dt, dev = x.dtype, x.device
    _dense("x", x, dt, (M, K), dev)
    for name, t in (("dg", dg), ("dfc", dfc)):
        _dense(name, t, dt, (M, N), dev)
    for name, t in (("w_g", w_g), ("w_fc", w_fc), ("dw_g", dw_g), ("dw_fc", dw_fc)):
        _dense(name, t, dt, (K, N), dev)
    _dense("dx", dx, dt, (M, K), dev)
    code = _dtype_code(x)
    nbytes = int(lib.swiglu_bwd_wx_workspace_size(M, K, N, code))
    with _on_device(dev):
        ws = _workspace(nbytes, workspace, dev, stream)
        st = lib.swiglu_bwd_wx(_ptr(x), _ptr(dg), _ptr(dfc), _ptr(w_g), _ptr(w_fc), _ptr(dw_g),
                               _ptr(dw_fc), _ptr(dx), M, K, N, code, _ptr(ws),
                               0 if ws is None else ws.numel() * ws.element_size(),
                               _stream(stream, dev))
    _check("swiglu_bwd_wx", st, lib)


def swiglu_fwd(x, w_g, w_fc, b_g, b_fc, g, fc, y, stream=None):
    """SwiGLU forward: g = x W_g + b_g, fc = x W_fc + b_fc, y = SiLU(g) fc (all three
    [M, N] outputs overwritten).  ``b_g`` / ``b_fc`` may be None (no bias)."""
    lib = load_library()
    if x.dim() != 2 or w_g.dim() != 2:
        raise ValueError("x must be [M, K] and w_g [K, N]")
    M, K = x.shape
    N = w_g.shape[1]
    dt, dev = x.dtype, x.device
    _dense("x", x, dt, (M, K), dev)
    for name, t in (("w_g", w_g), ("w_fc", w_fc)):
        _dense(name, t, dt, (K, N), dev)
    for name, t in (("b_g", b_g), ("b_fc", b_fc)):
        if t is not None:
            _dense(name, t, dt, (N,), dev)
    for name, t in (("g", g), ("fc", fc), ("y", y)):
        _dense(name, t, dt, (M, N), dev)
    with _on_device(dev):
        st = lib.swiglu_fwd(_ptr(x), _ptr(w_g), _ptr(w_fc), _ptr(b_g), _ptr(b_fc), _ptr(g),
                            _ptr(fc), _ptr(y), M, K, N, _dtype_code(x), _stream(stream, dev))
    _check("swiglu_fwd", st, lib)
