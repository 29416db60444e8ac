"""GPU parity of the SwiGLU forward entry point (through the C ABI) against the float64
oracle: the tiny and ragged workloads in full, odd shapes (partial row and column tiles,
contraction not a multiple of the stage depth), no bias, K = 0, fp16, guard bands, and
sampled rows of the large-batch shape."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import Guarded, device, note
from parity import U32, compare, forward_abs_models, sum_abs_model, to64
from workloads.gen import DTYPES, SWIGLU_WORKLOADS, SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu


def _sig(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-t))


def _fwd_case(inp, dt, bias=True, rows=None):
    dev = device()
    x, w_g, w_fc = inp["x"], inp["w_g"], inp["w_fc"]
    b_g, b_fc = (inp["b_g"], inp["b_fc"]) if bias else (None, None)
    M, K = x.shape
    N = w_g.shape[1]
    tdt = DTYPES[dt]
    g, fc, y = (Guarded((M, N), tdt, dev) for _ in range(3))
    note(f"forward M={M} K={K} N={N} {dt} bias={bias}")
    swg.swiglu_fwd(x.to(dev), w_g.to(dev), w_fc.to(dev),
                   None if b_g is None else b_g.to(dev), None if b_fc is None else b_fc.to(dev),
                   g.t, fc.t, y.t)
    torch.cuda.synchronize()
    for buf in (g, fc, y):
        buf.check()
    sel = slice(None) if rows is None else rows
    xr = to64(x[sel])
    zero = np.zeros(N)
    rg, rf, ry = R.swiglu_forward_ref(xr, to64(w_g), zero if b_g is None else to64(b_g),
                                      to64(w_fc), zero if b_fc is None else to64(b_fc))
    eg, ef, ey = forward_abs_models(xr, w_g, w_fc, b_g, b_fc, rg, rf)
    compare("g", g.t.cpu()[sel], rg, dt, model_abs=eg, contraction=K)
    compare("fc", fc.t.cpu()[sel], rf, dt, model_abs=ef, contraction=K)
    compare("y", y.t.cpu()[sel], ry, dt, model_abs=ey, contraction=K)
    return g.t, fc.t, y.t


@pytest.mark.parametrize("wl", ["tiny", "ragged"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_forward_workloads(wl, dt):
    _fwd_case(swiglu_inputs(wl, dtype=dt, with_forward=False), dt)


@pytest.mark.parametrize("M,K,N", [(1, 8, 8), (63, 72, 136), (300, 264, 264), (257, 520, 8),
                                   (700, 256, 128), (513, 1032, 72), (2000, 64, 2048),
                                   (300, 96, 64), (520, 384, 256)])
def test_forward_odd_shapes(M, K, N):
    inp = swiglu_inputs(SwiGLUShape("odd", 17, M, K, N), with_forward=False)
    _fwd_case(inp, "bf16")


@pytest.mark.parametrize("M,K,N", [(1, 4, 4), (63, 36, 132), (300, 260, 268), (257, 516, 12)])
def test_forward_fp32_odd_shapes(M, K, N):
    inp = swiglu_inputs(SwiGLUShape("odd32", 18, M, K, N), dtype="fp32", with_forward=False)
    _fwd_case(inp, "fp32")


@pytest.mark.parametrize("seed", range(8))
def test_forward_random_shapes(seed):
    """Seeded random shapes, bf16 / fp16 / fp32 in turn (K, N multiples of 8 or 4)."""
    dt = ("bf16", "fp16", "fp32")[seed % 3]
    vec = 4 if dt == "fp32" else 8
    rng = np.random.default_rng(2000 + seed)
    M = int(rng.integers(1, 3000))
    K = int(rng.integers(0, 1100 // vec + 1)) * vec
    N = int(rng.integers(1, 1100 // vec + 1)) * vec
    inp = swiglu_inputs(SwiGLUShape("frand", 80 + seed, M, max(K, vec), N), dtype=dt,
                        with_forward=False)
    if K == 0:
        inp["x"] = inp["x"][:, :0]
        inp["w_g"], inp["w_fc"] = inp["w_g"][:0], inp["w_fc"][:0]
    _fwd_case(inp, dt, bias=seed % 4 != 3)


def test_forward_without_bias():
    _fwd_case(swiglu_inputs(SwiGLUShape("nobias", 5, 777, 136, 264), with_forward=False),
              "bf16", bias=False)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_forward_empty_contraction_gives_bias_terms(dt):
    dev = device()
    M, N = 40, 24
    tdt = DTYPES[dt]
    b_g = torch.linspace(-3, 3, N).to(tdt)
    b_fc = torch.linspace(2, -1, N).to(tdt)
    g, fc, y = (torch.full((M, N), 7.0, dtype=tdt, device=dev) for _ in range(3))
    e = torch.empty(M, 0, dtype=tdt, device=dev)
    w = torch.empty(0, N, dtype=tdt, device=dev)
    note(f"forward K=0 {dt}")
    swg.swiglu_fwd(e, w, w, b_g.to(dev), b_fc.to(dev), g, fc, y)
    torch.cuda.synchronize()
    bg, bf = to64(b_g), to64(b_fc)
    want_y = bg * _sig(bg) * bf
    for name, got, want in (("g", g, bg), ("fc", fc, bf), ("y", y, want_y)):
        compare(name, got.cpu(), np.broadcast_to(want, (M, N)), dt,
                model_abs=np.broadcast_to(8.0 * U32 * np.abs(want), (M, N)))


def test_forward_feeds_backward_b_stage():
    """g and fc from the GPU forward are what the b stage consumes: the chained result
    matches the oracle b stage run on the same (GPU-rounded) g and fc."""
    dev = device()
    inp = swiglu_inputs("ragged", with_forward=False)
    g, fc, _ = _fwd_case(inp, "bf16")
    M, N = g.shape
    dy = inp["dy"].to(dev)
    dg, dfc = torch.empty_like(g), torch.empty_like(g)
    db_g = torch.zeros(N, dtype=torch.bfloat16, device=dev)
    db_fc = torch.zeros_like(db_g)
    note("forward -> b stage")
    swg.swiglu_bwd_b(dy, g, fc, dg, dfc, db_g, db_fc)
    torch.cuda.synchronize()
    rdg, rdfc, rdbg, rdbf = R.b_ref(to64(inp["dy"]), to64(g), to64(fc))
    compare("dg", dg.cpu(), rdg, "bf16")
    compare("dfc", dfc.cpu(), rdfc, "bf16")
    compare("db_g", db_g.cpu(), rdbg, "bf16",
            model_abs=sum_abs_model(np.abs(rdg).sum(axis=0)))


def test_forward_large_batch_sampled_rows():
    """The large-batch shape (M = 220000): every output at 2048 sampled rows, including the
    first and the last rows (the partial last row tile)."""
    shape = SWIGLU_WORKLOADS["ffn_220k"]
    inp = swiglu_inputs(shape, with_forward=False)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, shape.M - 1, shape.M - 2],
                                     rng.choice(shape.M, 2044, replace=False)]))
    _fwd_case(inp, "bf16", rows=torch.from_numpy(rows))


def test_forward_bitwise_deterministic():
    dev = device()
    inp = swiglu_inputs("ragged", with_forward=False)
    args = [inp[k].to(dev) for k in ("x", "w_g", "w_fc", "b_g", "b_fc")]
    M, N = inp["x"].shape[0], inp["w_g"].shape[1]
    outs = []
    for _ in range(2):
        o = [torch.empty(M, N, dtype=torch.bfloat16, device=dev) for _ in range(3)]
        note("forward rerun")
        swg.swiglu_fwd(*args, *o)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16).cpu() for t in o])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
