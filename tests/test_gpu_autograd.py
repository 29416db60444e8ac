"""The autograd wrapper (forward and backward in the library's kernels) element by element
against the float64 oracle, and normwise against float64 autograd of the same SwiGLU gate
on the CPU: every gradient, leading batch dimensions, no-bias and frozen-input cases.

Oracle parity: y, g and fc against ``swiglu_forward_ref`` on the wrapper's inputs; the five
gradients against ``swiglu_bwd_ref`` fed the g and fc the wrapper saved for its backward
(so the forward's rounding of g and fc does not enter the backward comparison), with the
rounding models of the stages: fp32 sums for db, one storage rounding of the b stage's dg
and dfc plus fp32 accumulation for dw and dx."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
from gpu_util import device, note
from parity import U32, chained_abs_model, compare, sum_abs_model, to64
from swish_activation_backward_amd.autograd import SwiGLU, swiglu
from workloads.gen import SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu

DT_NAME = {torch.bfloat16: "bf16", torch.float16: "fp16", torch.float32: "fp32"}


def _sig(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def _saved_g_fc(y):
    """The g and fc the wrapper saved for its backward (read before backward frees them);
    ``y`` is the wrapped function's output or a view of it."""
    out = y if y._base is None else y._base
    saved = out.grad_fn.saved_tensors        # (x, w_g, w_fc, g, fc)
    return saved[3], saved[4]


def _oracle_parity(y, saved, x, w_g, w_fc, b_g, b_fc, dy, grads):
    """y, the saved g / fc and the gradients (dict name -> tensor or None) element by
    element against the oracle."""
    dt = DT_NAME[y.dtype]
    y = y.detach()
    g_s, fc_s = to64(saved[0]), to64(saved[1])
    x64, wg64, wf64, dy64 = to64(x), to64(w_g), to64(w_fc), to64(dy)
    N = wg64.shape[1]
    bg64 = np.zeros(N) if b_g is None else to64(b_g)
    bf64 = np.zeros(N) if b_fc is None else to64(b_fc)
    rg, rf, ry = R.swiglu_forward_ref(x64, wg64, bg64, wf64, bf64)
    ax = np.abs(x64)
    eg = sum_abs_model(ax @ np.abs(wg64) + np.abs(bg64))
    ef = sum_abs_model(ax @ np.abs(wf64) + np.abs(bf64))
    s = _sig(rg)
    ey = (np.abs(s + rg * s * (1 - s)) * np.abs(rf) * eg + np.abs(rg * s) * ef
          + 8.0 * U32 * np.abs(rg * s * rf))
    K = wg64.shape[0]
    M = x64.reshape(-1, K).shape[0]
    compare("y", y, ry, dt, model_abs=ey, contraction=K)
    compare("saved g", g_s, rg, dt, model_abs=eg, contraction=K)
    compare("saved fc", fc_s, rf, dt, model_abs=ef, contraction=K)
    ref = R.swiglu_bwd_ref(dy64, x64, wg64, wf64, g_s, fc_s)
    adg, adfc = np.abs(ref["dg"]), np.abs(ref["dfc"])
    models = {"dx": chained_abs_model(adg @ np.abs(wg64).T + adfc @ np.abs(wf64).T, dt),
              "dw_g": chained_abs_model(ax.T @ adg, dt),
              "dw_fc": chained_abs_model(ax.T @ adfc, dt),
              "db_g": sum_abs_model(adg.sum(0)), "db_fc": sum_abs_model(adfc.sum(0))}
    terms = {"dx": 2 * N, "dw_g": M, "dw_fc": M, "db_g": M, "db_fc": M}
    for name, got in grads.items():
        if got is not None:
            compare(f"autograd {name}", got, ref[name], dt, model_abs=models[name],
                    contraction=terms[name])


def _ref_grads(x, w_g, w_fc, b_g, b_fc, dy):
    leaves = [t.double().requires_grad_() if t is not None else None
              for t in (x, w_g, w_fc, b_g, b_fc)]
    xx, wg, wf, bg, bf = leaves
    g = xx @ wg + (0 if bg is None else bg)
    fc = xx @ wf + (0 if bf is None else bf)
    y = torch.nn.functional.silu(g) * fc
    y.backward(dy.double())
    return y.detach(), [None if t is None else t.grad for t in leaves]


def _close(name, got, want, rel=2.0 ** -6):
    """Normwise: a correct bf16 pipeline (bf16 g, fc, dg, dfc between the stages) stays far
    inside 2^-6 relative error; a misplaced or missing term does not."""
    got = got.detach().cpu().double()
    err = (got - want).norm().item()
    assert err <= rel * want.norm().item() + 1e-30, f"{name}: {err} vs {want.norm().item()}"


@pytest.mark.parametrize("bias", [True, False])
def test_autograd_matches_float64_autograd(bias):
    dev = device()
    inp = swiglu_inputs(SwiGLUShape("ag", 21, 1000, 136, 264))
    x, w_g, w_fc = inp["x"], inp["w_g"], inp["w_fc"]
    b_g, b_fc = (inp["b_g"], inp["b_fc"]) if bias else (None, None)
    dy = inp["dy"]
    ref_y, ref = _ref_grads(x, w_g, w_fc, b_g, b_fc, dy)
    params = [t.to(dev).requires_grad_() if t is not None else None
              for t in (x, w_g, w_fc, b_g, b_fc)]
    note(f"autograd wrapper bias={bias}")
    y = swiglu(*params)
    saved = _saved_g_fc(y)
    y.backward(dy.to(dev))
    torch.cuda.synchronize()
    _oracle_parity(y, saved, x, w_g, w_fc, b_g, b_fc, dy,
                   {n: (None if p is None else p.grad) for n, p in
                    zip(("dx", "dw_g", "dw_fc", "db_g", "db_fc"), params)})
    _close("y", y, ref_y)
    for name, p, r in zip(("dx", "dw_g", "dw_fc", "db_g", "db_fc"), params, ref):
        if p is None:
            continue
        _close(name, p.grad, r)


def test_module_with_leading_dims_and_frozen_input():
    dev = device()
    torch.manual_seed(0)
    mod = SwiGLU(64, 128, device=dev)
    x = (torch.randn(3, 50, 64) / 8).to(torch.bfloat16).to(dev)   # input needs no grad
    note("autograd module [3, 50, 64] -> [3, 50, 128]")
    y = mod(x)
    assert y.shape == (3, 50, 128)
    saved = _saved_g_fc(y)
    dy = (torch.randn(3, 50, 128) / 8).to(torch.bfloat16)
    y.backward(dy.to(dev))
    torch.cuda.synchronize()
    ref_y, ref = _ref_grads(x.cpu().reshape(-1, 64), mod.w_g.detach().cpu(),
                            mod.w_fc.detach().cpu(), mod.b_g.detach().cpu(),
                            mod.b_fc.detach().cpu(), dy.reshape(-1, 128))
    # the [150, 128] output of the wrapped function (the module only reshapes around it)
    _oracle_parity(y.reshape(-1, 128), saved,
                   x.reshape(-1, 64), mod.w_g.detach(), mod.w_fc.detach(), mod.b_g.detach(),
                   mod.b_fc.detach(), dy.reshape(-1, 128),
                   {"dw_g": mod.w_g.grad, "dw_fc": mod.w_fc.grad, "db_g": mod.b_g.grad,
                    "db_fc": mod.b_fc.grad})
    _close("y", y.reshape(-1, 128), ref_y)
    for name, p, r in zip(("dw_g", "dw_fc", "db_g", "db_fc"),
                          (mod.w_g, mod.w_fc, mod.b_g, mod.b_fc), ref[1:]):
        _close(name, p.grad, r)


def test_autograd_fp32_end_to_end():
    """fp32 parameters: forward, b, w and x in the fp32 kernels; no 16-bit rounding between
    the stages, so the normwise agreement with float64 autograd is far tighter."""
    dev = device()
    inp = swiglu_inputs(SwiGLUShape("ag32", 22, 777, 132, 196), dtype="fp32")
    x, w_g, w_fc, b_g, b_fc, dy = (inp[k] for k in ("x", "w_g", "w_fc", "b_g", "b_fc", "dy"))
    ref_y, ref = _ref_grads(x, w_g, w_fc, b_g, b_fc, dy)
    params = [t.to(dev).requires_grad_() for t in (x, w_g, w_fc, b_g, b_fc)]
    note("autograd wrapper fp32")
    y = swiglu(*params)
    saved = _saved_g_fc(y)
    y.backward(dy.to(dev))
    torch.cuda.synchronize()
    _oracle_parity(y, saved, x, w_g, w_fc, b_g, b_fc, dy,
                   {n: p.grad for n, p in zip(("dx", "dw_g", "dw_fc", "db_g", "db_fc"), params)})
    _close("y", y, ref_y, rel=2.0 ** -16)
    for name, p, r in zip(("dx", "dw_g", "dw_fc", "db_g", "db_fc"), params, ref):
        _close(name, p.grad, r, rel=2.0 ** -16)

