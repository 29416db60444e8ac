"""Comparison rules between a GPU result and the float64 oracle (test infrastructure).

Three checks are applied to every output tensor:

1. the stated tolerance: |gpu - ref| <= atol + rtol * |ref| (numpy assert_allclose
   semantics).  For bf16 outputs this is the SwiGLU page's own check, rtol = 2^-7
   (bf16 machine epsilon) and atol = 1e-4 (section "精度校验", precision check).
   fp16 and fp32 results take rtol 1e-3 and 1e-5; because a rtol-only rule fails
   correct fp32-arithmetic kernels near the zero of s' and on fp16 subnormals, their
   atol is the rounding model of a correct fp32 evaluation (``swish_abs_model``);
2. a per-element mixed bound |gpu - ref| <= rtol * |ref| + E, where E is the
   rounding model of the arithmetic that produced the value (fp32 math + one final
   rounding).  This binds where atol = 1e-4 exceeds the outputs themselves;
3. a normwise bound ||gpu - ref||_2 <= nw * ||ref||_2.
"""
from __future__ import annotations

import numpy as np
import torch

U32 = 2.0 ** -24          # fp32 unit roundoff
BF16_RTOL = 2.0 ** -7     # bf16 machine epsilon: the SwiGLU page's rtol
BF16_ATOL = 1e-4          # the SwiGLU page's atol
FP16_RTOL = 1e-3
FP32_RTOL = 1e-5
FP16_SUBNORMAL_HALF = 2.0 ** -25

RTOL = {"bf16": BF16_RTOL, "fp16": FP16_RTOL, "fp32": FP32_RTOL}
NORMWISE = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10, "fp32": 2.0 ** -20}


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _sig(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def swish_abs_model(grad, x, beta):
    """Absolute error of a correct fp32 evaluation of grad*s'(beta x):
    8 * 2^-24 * |grad| * (sigma(t) + |t| sigma(t) (1 - sigma(t))), t = beta x."""
    t = float(np.float32(1.0 if beta is None else beta)) * to64(x)
    s = _sig(t)
    return 8.0 * U32 * np.abs(to64(grad)) * (s + np.abs(t) * s * (1.0 - s))


def dg_abs_model(dy, g, fc):
    g = to64(g)
    s = _sig(g)
    return 8.0 * U32 * np.abs(to64(dy) * to64(fc)) * (s + np.abs(g) * s * (1.0 - s))


def dfc_abs_model(dy, g):
    g = to64(g)
    return 8.0 * U32 * np.abs(to64(dy) * g * _sig(g))


def sum_abs_model(abs_sum):
    """fp32 accumulation of a sum whose magnitude sum is ``abs_sum``."""
    return 2.0 ** -16 * abs_sum


class ParityError(AssertionError):
    pass


def compare(name, gpu, ref, dtype, *, model_abs=None, atol=None, rtol=None,
            normwise=None, raise_on_fail=True):
    """Apply the three checks; return a stats dict (and raise on failure)."""
    g = to64(gpu)
    r = to64(ref)
    if g.shape != r.shape:
        raise ParityError(f"{name}: shape {g.shape} != {r.shape}")
    rtol = RTOL[dtype] if rtol is None else rtol
    nw = NORMWISE[dtype] if normwise is None else normwise
    if atol is None:
        if dtype == "bf16":
            atol = BF16_ATOL
        else:
            atol = 0.0 if model_abs is None else model_abs
            if dtype == "fp16":
                atol = atol + FP16_SUBNORMAL_HALF
    err = np.abs(g - r)
    absr = np.abs(r)
    stats = {"name": name, "n": int(r.size)}
    bad_nonfinite = int((~np.isfinite(g)).sum())
    stats["nonfinite"] = bad_nonfinite
    contract_bad = err > atol + rtol * absr
    stats["contract_fail"] = int(contract_bad.sum())
    if model_abs is not None:
        extra = FP16_SUBNORMAL_HALF if dtype == "fp16" else 0.0
        mixed_bad = err > rtol * absr + model_abs + extra
        stats["mixed_fail"] = int(mixed_bad.sum())
    else:
        stats["mixed_fail"] = 0
    nr = float(np.sqrt(np.sum(r * r)))
    ne = float(np.sqrt(np.sum(err * err)))
    stats["normwise"] = ne / nr if nr > 0 else ne
    normwise_bad = (ne > nw * nr) if nr > 0 else (ne > 0)
    stats["normwise_fail"] = bool(normwise_bad)
    stats["max_abs_err"] = float(err.max()) if err.size else 0.0
    ok = (bad_nonfinite == 0 and stats["contract_fail"] == 0 and stats["mixed_fail"] == 0
          and not normwise_bad)
    stats["ok"] = ok
    if raise_on_fail and not ok:
        idx = int(np.argmax(err - rtol * absr)) if err.size else 0
        raise ParityError(
            f"{name}: {stats}; worst at flat index {idx}: gpu={g.flat[idx]!r} "
            f"ref={r.flat[idx]!r}")
    return stats
