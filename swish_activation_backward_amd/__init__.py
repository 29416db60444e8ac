"""MI355X (gfx950) SwiGLU backward with the beta-scaled Swish gradient at its core.

The computation lives in ``libswiglu_bwd.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/swiglu_bwd.h``); this package is its thin ctypes binding.  The
binding loads the library lazily on first use and raises if it is missing.
"""
from ._lib import (  # noqa: F401
    DTYPE_CODE, STATUS, SwgError, library_path, load_library, swg_set_gemm_tile,
    swg_time_next_call, swg_version, swiglu_bwd_b, swiglu_bwd_b_noalloc,
    swiglu_bwd_b_workspace_size, swiglu_bwd_gemm_tile, swiglu_bwd_w, swiglu_bwd_w_workspace_size,
    swiglu_bwd_wx, swiglu_bwd_wx_workspace_size, swiglu_bwd_x, swiglu_fwd, swish_grad,
    swish_grad_strided,
)

__version__ = "0.1.0"
