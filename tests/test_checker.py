"""Negative and positive controls for the parity checker (CPU only).

A correct result rounded once to the storage dtype (nearest, or any direction within
one ulp) must pass; zeros, +-2 % noise and errors hidden below atol = 1e-4 must fail.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
from parity import (Checker, ParityError, compare, dg_abs_model, dfc_abs_model,
                    swish_abs_model)


def _round(ref, dtype, mode="nearest"):
    t = torch.tensor(ref, dtype=torch.float64)
    if mode == "nearest":
        return t.to(dtype).to(torch.float64).numpy()
    # toward zero: drop the low bits of the float32 image, then narrow (bf16 only)
    f = t.to(torch.float32)
    bits = f.view(torch.int32) & ~0xFFFF
    return bits.view(torch.float32).to(torch.float64).numpy()


@pytest.fixture(scope="module")
def bstage():
    rng = np.random.default_rng(0)
    M, N = 512, 256
    # magnitudes like the large-batch FFN workload: |dg| ~ 2e-5, mostly below atol
    dy = rng.normal(0, 1 / np.sqrt(220000), (M, N))
    g = rng.normal(0, 0.03, (M, N))
    fc = rng.normal(0, 0.03, (M, N))
    dg, dfc, _, _ = R.b_ref(dy, g, fc)
    return dy, g, fc, dg, dfc


def test_rounded_results_pass(bstage):
    dy, g, fc, dg, dfc = bstage
    for mode in ("nearest", "toward_zero"):
        compare("dg", _round(dg, torch.bfloat16, mode), dg, "bf16", model_abs=dg_abs_model(dy, g, fc))
        compare("dfc", _round(dfc, torch.bfloat16, mode), dfc, "bf16", model_abs=dfc_abs_model(dy, g))


@pytest.mark.parametrize("bad", ["zeros", "noise2pct", "half_below_atol", "sign"])
def test_wrong_results_fail(bstage, bad):
    dy, g, fc, dg, dfc = bstage
    rng = np.random.default_rng(1)
    if bad == "zeros":
        out = np.zeros_like(dg)
    elif bad == "noise2pct":
        out = _round(dg * (1 + 0.02 * rng.choice([-1.0, 1.0], dg.shape)), torch.bfloat16)
    elif bad == "half_below_atol":
        # 50 % error wherever that stays below atol = 1e-4 (nearly every element)
        out = _round(np.where(np.abs(dg) < 1.8e-4, dg * 1.5, dg), torch.bfloat16)
        assert np.all(np.abs(out - dg) <= 1e-4 + 2 ** -7 * np.abs(dg))
    else:
        out = -dg
    with pytest.raises(ParityError):
        compare("dg", out, dg, "bf16", model_abs=dg_abs_model(dy, g, fc))


def test_fp32_swish_emulation_passes_and_wrong_beta_fails():
    rng = np.random.default_rng(2)
    x = (rng.normal(0, 3, 200000)).astype(np.float32)
    grad = rng.normal(0, 1, 200000).astype(np.float32)
    for beta in (1.0, 1.702, 0.5):
        ref = R.swish_grad_ref(grad, x, beta)
        # a float32 evaluation of the same formula (what a correct kernel does)
        t = np.float32(beta) * x
        with np.errstate(over="ignore"):
            s = (np.float32(1) / (np.float32(1) + np.exp(-t))).astype(np.float32)
        out = grad * (s + t * s * (np.float32(1) - s))
        compare("fp32", out, ref, "fp32", model_abs=swish_abs_model(grad, x, beta))
        out16 = torch.tensor(out).to(torch.float16)
        compare("fp16", out16, R.swish_grad_ref(grad, x, beta), "fp16",
                model_abs=swish_abs_model(grad, x, beta))
    wrong = R.swish_grad_ref(grad, x, 1.0001)
    with pytest.raises(ParityError):
        compare("fp32", wrong, R.swish_grad_ref(grad, x, 1.0), "fp32",
                model_abs=swish_abs_model(grad, x, 1.0))


def test_checker_accumulates_chunks(bstage):
    dy, g, fc, dg, dfc = bstage
    c = Checker("dg", "bf16")
    for i in range(0, dg.shape[0], 100):
        c.add(_round(dg[i:i + 100], torch.bfloat16), dg[i:i + 100],
              dg_abs_model(dy[i:i + 100], g[i:i + 100], fc[i:i + 100]))
    st = c.result()
    assert st["n"] == dg.size and st["ok"]
    c2 = Checker("dg", "bf16")
    c2.add(np.zeros_like(dg[:10]), dg[:10])
    with pytest.raises(ParityError):
        c2.result()


def test_fp32_contraction_normwise_bound():
    """fp32 outputs that sum n products get the normwise bound max(2^-20, 2 u sqrt(n));
    bf16 and fp16 keep their storage-rounding bounds.  A sum evaluated in fp32 (sequential,
    products rounded) over 3008 random-sign terms passes with it, while 1e-4 relative noise
    fails; the fixed fp32 bound stays 2^-20 for short sums."""
    from parity import NORMWISE, U32, contraction_normwise, sum_abs_model
    assert contraction_normwise("fp32", 16) == 2.0 ** -20
    assert contraction_normwise("fp32", 3008) == pytest.approx(2 * U32 * np.sqrt(3008))
    assert contraction_normwise("bf16", 10 ** 6) == NORMWISE["bf16"]
    assert contraction_normwise("fp16", 10 ** 6) == NORMWISE["fp16"]
    rng = np.random.default_rng(3)
    n, m = 3008, 400
    a = rng.normal(0, 1, (m, n)).astype(np.float32)
    b = rng.normal(0, 1, n).astype(np.float32)
    exact = a.astype(np.float64) @ b.astype(np.float64)
    acc = np.zeros(m, dtype=np.float32)
    for k in range(n):                        # fp32 products and fp32 running sums
        acc = (acc + a[:, k] * b[k]).astype(np.float32)
    model = sum_abs_model(np.abs(a.astype(np.float64)) @ np.abs(b.astype(np.float64)))
    assert compare("fp32 sum", acc.astype(np.float64), exact, "fp32", model_abs=model,
                   contraction=n)["ok"]
    noisy = exact * (1 + 1e-4 * rng.choice([-1.0, 1.0], m))
    with pytest.raises(ParityError):
        compare("fp32 sum, noisy", noisy, exact, "fp32", model_abs=model, contraction=n)
