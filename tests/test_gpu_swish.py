"""GPU parity of swish_grad (through the C ABI) against the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import Guarded, device, note
from parity import TORCH_NAME, compare, swish_abs_model
from workloads.gen import DTYPES, SWISH_CONTEXT, SWISH_WORKLOAD, swish_inputs

pytestmark = pytest.mark.gpu

_cache = {}


def _inputs(dt):
    if dt not in _cache:
        _cache.clear()
        _cache[dt] = swish_inputs(dt)
    return _cache[dt]


@pytest.mark.parametrize("dt", SWISH_WORKLOAD["dtypes"])
@pytest.mark.parametrize("beta", SWISH_WORKLOAD["betas"])
def test_swish_grad_full_length(dt, beta):
    """L = 2^24 + 37 (ragged tail), grad ~ N(0,1), x ~ N(0,3); every element compared."""
    dev = device()
    inp = _inputs(dt)
    grad, x = inp["grad"], inp["x"]
    note(f"swish_grad full L={grad.numel()} {dt} beta={beta}")
    gx = swg.swish_grad(grad.to(dev), x.to(dev), beta=beta)
    torch.cuda.synchronize()
    ref = R.swish_grad_ref(grad.double().numpy(), x.double().numpy(), beta)
    compare(f"swish_grad[{dt},{beta}]", gx.cpu(), ref, dt,
            model_abs=swish_abs_model(grad.double().numpy(), x.double().numpy(), beta))


def test_swish_grad_pages_timed_shape():
    """The fp16 [32, 64, 56, 56] activation the Ascend C page times (beta = 1, SiLU
    backward), as a 4-D contiguous tensor; every element compared."""
    dev = device()
    c = SWISH_CONTEXT
    L = int(np.prod(c["shape"]))
    inp = swish_inputs(c["dtype"], L=L, seed=c["seed"])
    grad, x = inp["grad"].reshape(c["shape"]), inp["x"].reshape(c["shape"])
    note(f"swish_grad {c['shape']} {c['dtype']} beta={c['beta']}")
    gx = swg.swish_grad(grad.to(dev), x.to(dev), beta=c["beta"])
    torch.cuda.synchronize()
    assert gx.shape == grad.shape
    g64, x64 = grad.reshape(-1).double().numpy(), x.reshape(-1).double().numpy()
    ref = R.swish_grad_ref(g64, x64, c["beta"])
    compare("swish_grad[32,64,56,56]", gx.reshape(-1).cpu(), ref, c["dtype"],
            model_abs=swish_abs_model(g64, x64, c["beta"]))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("n", [1, 5, 8, 13, 1000, 65541, 262151])
@pytest.mark.parametrize("beta", [None, 0.0, -1.3, 2.5, 0.01])
def test_swish_grad_small_and_ragged(dt, n, beta):
    dev = device()
    inp = swish_inputs(dt, L=n, seed=100 + n)
    g = Guarded((n,), DTYPES[dt], dev)
    note(f"swish_grad n={n} {dt} beta={beta}")
    swg.swish_grad(inp["grad"].to(dev), inp["x"].to(dev), grad_x=g.t, beta=beta)
    torch.cuda.synchronize()
    g.check()
    ref = R.swish_grad_ref(inp["grad"].double().numpy(), inp["x"].double().numpy(), beta)
    compare("swish_grad", g.t.cpu(), ref, dt,
            model_abs=swish_abs_model(inp["grad"].double().numpy(), inp["x"].double().numpy(), beta))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("which", ["grad", "x"])
def test_swish_grad_in_place(dt, which):
    dev = device()
    n = 100003
    inp = swish_inputs(dt, L=n, seed=7)
    ref = R.swish_grad_ref(inp["grad"].double().numpy(), inp["x"].double().numpy(), 1.702)
    grad, x = inp["grad"].to(dev), inp["x"].to(dev)
    out = grad if which == "grad" else x
    note(f"swish_grad in place on {which} {dt}")
    swg.swish_grad(grad, x, grad_x=out, beta=1.702)
    torch.cuda.synchronize()
    compare("swish_grad in place", out.cpu(), ref, dt,
            model_abs=swish_abs_model(inp["grad"].double().numpy(), inp["x"].double().numpy(), 1.702))


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_swish_grad_unaligned_pointers_take_scalar_path(dt):
    dev = device()
    n = 5000
    inp = swish_inputs(dt, L=n + 1, seed=9)
    grad = inp["grad"].to(dev)[1:]          # 2- or 4-byte offset: not 16-byte aligned
    x = inp["x"].to(dev)[1:]
    out = torch.empty(n + 1, dtype=DTYPES[dt], device=dev)[1:]
    note(f"swish_grad unaligned {dt}")
    swg.swish_grad(grad, x, grad_x=out, beta=0.5)
    torch.cuda.synchronize()
    ref = R.swish_grad_ref(inp["grad"][1:].double().numpy(), inp["x"][1:].double().numpy(), 0.5)
    compare("swish_grad unaligned", out.cpu(), ref, dt,
            model_abs=swish_abs_model(inp["grad"][1:].double().numpy(),
                                      inp["x"][1:].double().numpy(), 0.5))


def test_swish_grad_empty_and_saturation():
    dev = device()
    e = torch.empty(0, dtype=torch.bfloat16, device=dev)
    swg.swish_grad(e, e, grad_x=e)
    # extreme arguments: no NaN, limits 0 (t -> -inf) and grad (t -> +inf)
    x = torch.tensor([-1e4, -200.0, -90.0, 90.0, 200.0, 1e4, 0.0, -0.0], dtype=torch.float32)
    grad = torch.ones_like(x)
    note("swish_grad saturation")
    out = swg.swish_grad(grad.to(dev), x.to(dev), beta=1.0).cpu()
    ref = R.swish_grad_ref(grad.double().numpy(), x.double().numpy(), 1.0)
    assert torch.all(torch.isfinite(out))
    compare("saturation", out, ref, "fp32", model_abs=swish_abs_model(grad, x, 1.0))
    assert out[6].item() == 0.5 and out[7].item() == 0.5


def test_swish_grad_deterministic():
    dev = device()
    inp = swish_inputs("bf16", L=1 << 20, seed=3)
    g, x = inp["grad"].to(dev), inp["x"].to(dev)
    a = swg.swish_grad(g, x, beta=1.702)
    b = swg.swish_grad(g, x, beta=1.702)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
