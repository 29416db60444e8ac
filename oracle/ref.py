"""Plain float64 CPU oracle for the SwiGLU backward and the beta-scaled Swish gradient.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or run this
module: only the tests, the package's smoke check and the bench's CPU-baseline leg use
it.  It shares no code with the HIP kernels or their host library.

Every function is the plain mathematical definition written out in numpy float64,
with no blocking, fusion or reordering.  Inputs are the exact tensors the GPU
received, widened to float64 (exact for bf16, fp16 and fp32).  Sources:

  [SwiGLU page]  "PyPTO-Gym 实战: Fused SwiGLU 反向传播算子" (hnwysp.cn), section
                 "算法概述与数学公式" (algorithm overview and formulas), items 1-4,
                 and the SwiGLU forward in "算子背景" (operator background).
  [Swish page]   "CANN ops-nn 中 SwishGrad 算子解析" (bhfrc.com), section 1.2
                 "计算公式" (formula) and section 2.4 (kernel compute chain).
  [Ascend C page] "Ascend C 自定义反向算子" (cann.csdn.net), section 2.1 (math
                 definition of the Swish gradient).

Readings taken where the pages are garbled or silent:
  * The SwiGLU page's extracted formulas lost '=', '+' and the prime on SiLU'.  The
    gate gradient is read as dg = dy*fc*SiLU'(g) with SiLU'(g) = s(1 + g(1 - s)),
    s = sigmoid(g); the page's description of its code builds dg the same way (the
    product dy*fc times the SiLU derivative), and it is the derivative of g*sigmoid(g).
  * The sigmoid is 1/(1 + exp(-t)) (the Swish page's definition), which is finite for
    every finite t; the SwiGLU page's exp(g)/(1 + exp(g)) is the same function.
  * db and dw are accumulated into caller-provided buffers (the SwiGLU page says they
    must be zero-initialised because the kernels add into them); the oracle adds the
    initial value exactly.
  * beta is a float32 scalar on the Swish page; the oracle widens that float32 value.
"""
from __future__ import annotations

import numpy as np

__all__ = ["sigmoid", "silu", "silu_grad", "swish_grad_ref", "b_ref", "w_ref",
           "x_ref", "swiglu_forward_ref", "swiglu_bwd_ref"]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def sigmoid(t):
    """sigma(t) = 1 / (1 + exp(-t))  [Swish page, section 1.2, sigmoid definition].

    exp(-t) overflows to +inf for t < -709; 1/(1+inf) = 0 is then the correct limit.
    """
    t = _f64(t)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def silu(t):
    """SiLU(t) = t * sigma(t)  [SwiGLU page, operator background]."""
    t = _f64(t)
    return t * sigmoid(t)


def silu_grad(t):
    """d/dt SiLU(t) = sigma(t) * (1 + t * (1 - sigma(t)))  [SwiGLU page, formula 1]."""
    t = _f64(t)
    s = sigmoid(t)
    return s * (1.0 + t * (1.0 - s))


def swish_grad_ref(grad, x, beta=1.0):
    """grad_x = grad * s'(x),  s(x) = x * sigma(beta x),
    s'(x) = sigma(beta x) * (1 + beta x * (1 - sigma(beta x)))
    [Swish page, section 1.2, derivative of the Swish forward; Ascend C page, 2.1].

    ``beta`` is the float32 scalar the kernel receives (None means 1.0, as the Swish
    page's aclnn interface specifies for a missing beta).
    """
    b = 1.0 if beta is None else float(np.float32(beta))
    x = _f64(x)
    t = b * x
    s = sigmoid(t)
    return _f64(grad) * (s * (1.0 + t * (1.0 - s)))


def b_ref(dy, g, fc, db_g0=None, db_fc0=None):
    """b stage [SwiGLU page, formulas 1 and 2]:
        dg  = dy * fc * SiLU'(g)
        dfc = dy * SiLU(g) = dy * g * sigma(g)
        db_g  = db_g0  + sum over the batch dimension of dg
        db_fc = db_fc0 + sum over the batch dimension of dfc
    dy, g, fc: [M, N].  Returns (dg, dfc, db_g, db_fc) in float64.
    """
    dy, g, fc = _f64(dy), _f64(g), _f64(fc)
    N = dy.shape[-1]
    dg = dy * fc * silu_grad(g)
    dfc = dy * silu(g)
    db_g = (np.zeros(N) if db_g0 is None else _f64(db_g0).reshape(N)) + dg.sum(axis=0)
    db_fc = (np.zeros(N) if db_fc0 is None else _f64(db_fc0).reshape(N)) + dfc.sum(axis=0)
    return dg, dfc, db_g, db_fc


def w_ref(x, dg, dfc, dw_g0=None, dw_fc0=None):
    """w stage [SwiGLU page, formula 3]: dw_g = dw_g0 + x^T dg, dw_fc = dw_fc0 + x^T dfc.

    x: [M, K]; dg, dfc: [M, N].  Returns (dw_g, dw_fc), each [K, N] float64.
    """
    x, dg, dfc = _f64(x), _f64(dg), _f64(dfc)
    K, N = x.shape[1], dg.shape[1]
    dw_g = x.T @ dg
    dw_fc = x.T @ dfc
    if dw_g0 is not None:
        dw_g = dw_g + _f64(dw_g0).reshape(K, N)
    if dw_fc0 is not None:
        dw_fc = dw_fc + _f64(dw_fc0).reshape(K, N)
    return dw_g, dw_fc


def x_ref(dg, dfc, w_g, w_fc):
    """x stage [SwiGLU page, formula 4]: dx = dg W_g^T + dfc W_fc^T.

    dg, dfc: [M, N]; w_g, w_fc: [K, N].  Returns dx [M, K] float64.
    """
    dg, dfc, w_g, w_fc = _f64(dg), _f64(dfc), _f64(w_g), _f64(w_fc)
    return dg @ w_g.T + dfc @ w_fc.T


def swiglu_forward_ref(x, w_g, b_g, w_fc, b_fc):
    """SwiGLU forward [SwiGLU page, operator background]:
    Gate = x W_g + b_g, FC = x W_fc + b_fc, y = SiLU(Gate) * FC.
    Returns (g, fc, y) in float64 (no rounding)."""
    x = _f64(x)
    g = x @ _f64(w_g) + _f64(b_g)
    fc = x @ _f64(w_fc) + _f64(b_fc)
    return g, fc, silu(g) * fc


def swiglu_bwd_ref(dy, x, w_g, w_fc, g, fc):
    """All seven gradients of the three-stage backward, chained in float64
    (b, then w and x consume the unrounded dg and dfc)."""
    dg, dfc, db_g, db_fc = b_ref(dy, g, fc)
    dw_g, dw_fc = w_ref(x, dg, dfc)
    dx = x_ref(dg, dfc, w_g, w_fc)
    return {"dg": dg, "dfc": dfc, "db_g": db_g, "db_fc": db_fc,
            "dw_g": dw_g, "dw_fc": dw_fc, "dx": dx}
