"""Comparison rules between a GPU result and the float64 oracle (test infrastructure).

Three checks are applied to every output tensor:

1. the stated tolerance: |gpu - ref| <= atol + rtol * |ref| (numpy assert_allclose
   semantics).  For bf16 outputs this is the SwiGLU page's own check, rtol = 2^-7
   (bf16 machine epsilon) and atol = 1e-4 (section "精度校验", precision check).
   fp16 and fp32 results take rtol 1e-3 and 1e-5; because a rtol-only rule fails
   correct fp32-arithmetic kernels near the zero of s' and on fp16 subnormals, their
   atol is the rounding model of a correct fp32 evaluation (``*_abs_model``);
2. a per-element mixed bound |gpu - ref| <= rtol * |ref| + E, where E is the
   rounding model of the arithmetic that produced the value (fp32 math + one final
   rounding).  This binds where atol = 1e-4 exceeds the outputs themselves;
3. a normwise bound ||gpu - ref||_2 <= nw * ||ref||_2 (bf16: 2^-8, the unit roundoff of
   an 8-bit significand; a correctly rounded bf16 tensor sits near 0.4 * 2^-8), plus
   sqrt(n) * 2^-25 for fp16, whose subnormals (below 2^-14) are spaced 2^-24 apart so that
   a correctly rounded value may miss by half of that whatever its size.

``Checker`` accumulates the three over chunks so that large tensors can be compared
piecewise; ``compare`` is the one-shot form.
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
NORMWISE = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -10, "fp32": 2.0 ** -20}
# unit roundoff of each storage type (RNE): the relative error of one rounding
STORAGE_UNIT = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -24}
TORCH_NAME = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


def to64(t) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        return t.detach().cpu().to(torch.float64).numpy()
    return np.asarray(t, dtype=np.float64)


def _sig(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


FP32_TINY = 2.0 ** -126   # smallest normal fp32: hardware exp may flush below it
# Absolute floor of a correct result's last rounding below the smallest normal: half the
# fp16 subnormal spacing; for fp32, a result under 2^-126 rounded to the subnormal grid
# (error <= 2^-150) or flushed to zero (error < 2^-126).  bf16 results carry atol 1e-4.
SUBNORMAL_FLOOR = {"bf16": 0.0, "fp16": FP16_SUBNORMAL_HALF, "fp32": FP32_TINY}


def swish_abs_model(grad, x, beta):
    """Absolute error of a correct fp32 evaluation of grad*s'(beta x):
    8 * 2^-24 * |grad| * (sigma(t) + |t| sigma(t) (1 - sigma(t))), t = beta x, plus
    |grad| (1 + |t|) 2^-126 for an exp(-|t|) flushed to zero below the fp32 normals."""
    t = float(np.float32(1.0 if beta is None else beta)) * to64(x)
    s = _sig(t)
    ag = np.abs(to64(grad))
    return 8.0 * U32 * ag * (s + np.abs(t) * s * (1.0 - s)) + ag * (1.0 + np.abs(t)) * FP32_TINY


def dg_abs_model(dy, g, fc):
    g = to64(g)
    s = _sig(g)
    a = np.abs(to64(dy) * to64(fc))
    return 8.0 * U32 * a * (s + np.abs(g) * s * (1.0 - s)) + a * (1.0 + np.abs(g)) * FP32_TINY


def dfc_abs_model(dy, g):
    g = to64(g)
    a = np.abs(to64(dy) * g)
    return 8.0 * U32 * a * _sig(g) + a * FP32_TINY


def sum_abs_model(abs_sum):
    """fp32 accumulation of a sum whose magnitude sum is ``abs_sum``."""
    return 2.0 ** -16 * np.asarray(abs_sum, dtype=np.float64)


def forward_abs_models(x, w_g, w_fc, b_g, b_fc, g, fc):
    """Rounding models of a correct kernel: fp32 accumulation of g and fc (2^-16 times the
    magnitude sums, bias included) and their propagation into y = g sigma(g) fc, plus the
    fp32 evaluation of y itself."""
    ax = np.abs(to64(x))
    ag = ax @ np.abs(to64(w_g)) + (0.0 if b_g is None else np.abs(to64(b_g)))
    af = ax @ np.abs(to64(w_fc)) + (0.0 if b_fc is None else np.abs(to64(b_fc)))
    eg, ef = sum_abs_model(ag), sum_abs_model(af)
    s = _sig(g)
    ds = np.abs(s + g * s * (1.0 - s))          # d SiLU / d g
    ey = ds * np.abs(fc) * eg + np.abs(g * s) * ef + 8.0 * U32 * np.abs(g * s * fc)
    return eg, ef, ey


def chained_abs_model(abs_sum, dtype):
    """A sum of products whose operand was itself a rounded output of an earlier stage
    (the w and x stages fed by the b stage's dg and dfc, stored in ``dtype``): each operand
    element carries a relative error of at most the storage unit roundoff u, so the
    result moves by at most u * A on top of the fp32 accumulation, A the magnitude sum."""
    return (STORAGE_UNIT[dtype] + 2.0 ** -16) * np.asarray(abs_sum, dtype=np.float64)


class ParityError(AssertionError):
    pass


def contraction_normwise(dtype, n):
    """Normwise bound of an output that sums ``n`` products.  bf16 and fp16 results are
    dominated by their storage rounding (the fixed bounds).  An fp32 result's rounding in
    the fp32 accumulation grows with the number of terms like a random walk: relative to
    the result's norm, about u sqrt(n) for sums whose terms cancel (random signs), so the
    fp32 bound is max(2^-20, 2 u sqrt(n))."""
    nw = NORMWISE[dtype]
    if dtype == "fp32" and n is not None and n > 0:
        nw = max(nw, 2.0 * U32 * float(np.sqrt(n)))
    return nw


class Checker:
    def __init__(self, name, dtype, *, rtol=None, atol=None, normwise=None, contraction=None):
        self.name, self.dtype = name, dtype
        self.rtol = RTOL[dtype] if rtol is None else rtol
        self.atol = atol
        self.nw = contraction_normwise(dtype, contraction) if normwise is None else normwise
        self.n = self.nonfinite = self.contract_fail = self.mixed_fail = 0
        self.ss_ref = self.ss_err = 0.0
        self.max_abs_err = 0.0
        self.worst = None
        self.worst_excess = -np.inf

    def add(self, gpu, ref, model_abs=None):
        g, r = to64(gpu), to64(ref)
        if g.shape != r.shape:
            raise ParityError(f"{self.name}: shape {g.shape} != {r.shape}")
        err = np.abs(g - r)
        absr = np.abs(r)
        if self.atol is not None:
            atol = self.atol
        elif self.dtype == "bf16":
            atol = BF16_ATOL
        else:
            atol = 0.0 if model_abs is None else model_abs
            atol = atol + SUBNORMAL_FLOOR[self.dtype]
        self.n += r.size
        self.nonfinite += int((~np.isfinite(g)).sum())
        self.contract_fail += int((err > atol + self.rtol * absr).sum())
        if model_abs is not None:
            bound = self.rtol * absr + model_abs + SUBNORMAL_FLOOR[self.dtype]
            self.mixed_fail += int((err > bound).sum())
        self.ss_ref += float(np.sum(r * r))
        self.ss_err += float(np.sum(err * err))
        if err.size:
            self.max_abs_err = max(self.max_abs_err, float(err.max()))
            ex = err - self.rtol * absr
            i = int(np.argmax(ex))
            if ex.flat[i] > self.worst_excess:
                self.worst_excess = float(ex.flat[i])
                self.worst = (float(g.flat[i]), float(r.flat[i]))
        return self

    def merge(self, other):
        """Fold in another Checker's counts (chunks checked on other threads)."""
        for k in ("n", "nonfinite", "contract_fail", "mixed_fail"):
            setattr(self, k, getattr(self, k) + getattr(other, k))
        self.ss_ref += other.ss_ref
        self.ss_err += other.ss_err
        self.max_abs_err = max(self.max_abs_err, other.max_abs_err)
        if other.worst_excess > self.worst_excess:
            self.worst_excess, self.worst = other.worst_excess, other.worst
        return self

    def result(self, raise_on_fail=True):
        nr, ne = np.sqrt(self.ss_ref), np.sqrt(self.ss_err)
        normwise = ne / nr if nr > 0 else ne
        floor = np.sqrt(self.n) * FP16_SUBNORMAL_HALF if self.dtype == "fp16" else 0.0
        normwise_bad = (ne > self.nw * nr + floor) if nr > 0 else (ne > floor)
        stats = {"name": self.name, "n": self.n, "nonfinite": self.nonfinite,
                 "contract_fail": self.contract_fail, "mixed_fail": self.mixed_fail,
                 "normwise": float(normwise), "normwise_fail": bool(normwise_bad),
                 "max_abs_err": self.max_abs_err}
        ok = (self.nonfinite == 0 and self.contract_fail == 0 and self.mixed_fail == 0
              and not normwise_bad)
        stats["ok"] = ok
        if raise_on_fail and not ok:
            raise ParityError(f"{self.name}: {stats}; worst (gpu, ref) = {self.worst}")
        return stats


def compare(name, gpu, ref, dtype, *, model_abs=None, atol=None, rtol=None,
            normwise=None, contraction=None, raise_on_fail=True):
    """Apply the three checks to one tensor; return a stats dict (raise on failure).
    ``contraction``: the number of products each output element sums (GEMM outputs and
    column sums), which sets the fp32 normwise bound (contraction_normwise)."""
    return Checker(name, dtype, rtol=rtol, atol=atol, normwise=normwise,
                   contraction=contraction).add(gpu, ref, model_abs).result(raise_on_fail)
