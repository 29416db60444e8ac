"""GPU parity of the fused w + x pass (swiglu_bwd_wx, through the C ABI) against the
float64 oracle: tiny and ragged workloads, odd and seeded random shapes (partial tiles,
one or several M splits), bf16 and fp16, accumulation into a non-zero dW, guard bands,
dx bit-identical to the x stage and dW equal to the w stage within the rounding model.
The full-size workloads are in test_gpu_full.py."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import Guarded, device, note, oracle_b_chunked, oracle_w_chunked, oracle_x_rows
from parity import compare, sum_abs_model, to64
from workloads.gen import DTYPES, SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu


def _oracle_dg(inp, dt):
    res = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], store_dtype=DTYPES[dt])
    return res["dg"], res["dfc"]


def _fused_case(inp, dt, dw0=None):
    dev = device()
    x, w_g, w_fc = inp["x"], inp["w_g"], inp["w_fc"]
    dg, dfc = _oracle_dg(inp, dt)
    M, K = x.shape
    N = dg.shape[1]
    tdt = DTYPES[dt]
    init = torch.zeros(K, N, dtype=tdt) if dw0 is None else dw0
    dw_g = Guarded((K, N), tdt, dev, fill=init.to(dev))
    dw_fc = Guarded((K, N), tdt, dev, fill=(2 * init).to(dev))
    dx = Guarded((M, K), tdt, dev)
    d = {k: v.to(dev) for k, v in (("x", x), ("dg", dg), ("dfc", dfc), ("w_g", w_g),
                                   ("w_fc", w_fc))}
    note(f"fused w+x M={M} K={K} N={N} {dt} init={'zero' if dw0 is None else 'nonzero'}")
    swg.swiglu_bwd_wx(d["x"], d["dg"], d["dfc"], d["w_g"], d["w_fc"], dw_g.t, dw_fc.t, dx.t)
    torch.cuda.synchronize()
    for buf in (dw_g, dw_fc, dx):
        buf.check()
    # the separate stages on the same inputs
    sep_dx = torch.empty(M, K, dtype=tdt, device=dev)
    sep_g, sep_fc = init.to(dev).clone(), (2 * init).to(dev).clone()
    swg.swiglu_bwd_x(d["dg"], d["dfc"], d["w_g"], d["w_fc"], sep_dx)
    swg.swiglu_bwd_w(d["x"], d["dg"], d["dfc"], sep_g, sep_fc)
    torch.cuda.synchronize()
    assert torch.equal(dx.t.cpu().view(torch.int16), sep_dx.cpu().view(torch.int16)), "dx"
    # oracle parity of every output
    rg, rf, ag, af = oracle_w_chunked(x, dg, dfc)
    i64 = to64(init)
    compare("fused dw_g", dw_g.t.cpu(), rg + i64, dt, model_abs=sum_abs_model(ag + np.abs(i64)))
    compare("fused dw_fc", dw_fc.t.cpu(), rf + 2 * i64, dt,
            model_abs=sum_abs_model(af + 2 * np.abs(i64)))
    ref, a = oracle_x_rows(dg, dfc, w_g, w_fc, slice(None))
    compare("fused dx", dx.t.cpu(), ref, dt, model_abs=sum_abs_model(a))
    # dW against the w stage: both within one rounding of each other's exact sums
    compare("fused dw_g vs w stage", dw_g.t.cpu(), sep_g.cpu(), dt,
            model_abs=2 * sum_abs_model(ag + np.abs(i64)))


@pytest.mark.parametrize("wl", ["tiny", "ragged"])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_fused_workloads(wl, dt, tile):
    _fused_case(swiglu_inputs(wl, dtype=dt), dt)


def test_fused_accumulates_into_nonzero_dw():
    inp = swiglu_inputs("ragged", dtype="bf16")
    K, N = inp["w_g"].shape
    dw0 = (torch.randn(K, N, generator=torch.Generator().manual_seed(9)) * 1e-3).to(torch.bfloat16)
    _fused_case(inp, "bf16", dw0=dw0)


@pytest.mark.parametrize("M,K,N", [(1, 8, 8), (63, 72, 136), (300, 264, 264), (1000, 8, 520),
                                   (257, 520, 8), (700, 256, 128), (513, 1032, 72),
                                   (2000, 64, 2048), (4099, 256, 256), (20000, 512, 64)])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_fused_odd_shapes(M, K, N, dt, tile):
    _fused_case(swiglu_inputs(SwiGLUShape("fodd", 23, M, K, N), dtype=dt), dt)


@pytest.mark.parametrize("seed", range(8))
def test_fused_random_shapes(seed, tile):
    rng = np.random.default_rng(3000 + seed)
    M = int(rng.integers(1, 12000))
    K = int(rng.integers(1, 1100 // 8 + 1)) * 8
    N = int(rng.integers(1, 1100 // 8 + 1)) * 8
    dt = "bf16" if seed % 2 == 0 else "fp16"
    _fused_case(swiglu_inputs(SwiGLUShape("frand", 80 + seed, M, K, N), dtype=dt), dt)


def test_fused_empty_contraction_and_fp32():
    dev = device()
    M, K = 33, 16
    bf = torch.bfloat16
    dx = torch.full((M, K), 3.0, dtype=bf, device=dev)
    e = torch.empty(M, 0, dtype=bf, device=dev)
    w = torch.empty(K, 0, dtype=bf, device=dev)
    x = torch.ones(M, K, dtype=bf, device=dev)
    note("fused w+x N=0")
    swg.swiglu_bwd_wx(x, e, e, w, w, w.clone(), w.clone(), dx)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0
    f = torch.float32
    with pytest.raises(swg.SwgError):
        swg.swiglu_bwd_wx(x.to(f), e.to(f), e.to(f), w.to(f), w.to(f), w.to(f), w.to(f), dx.to(f))
