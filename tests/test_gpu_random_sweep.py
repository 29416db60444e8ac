"""Seeded random sweep through every SwiGLU entry point: the b stage, the w and x stages,
the fused w + x pass and the forward at random shapes (M from 1 to 6000, K and N up to
1536, some of them a single vector wide), dtypes (bf16, fp16, fp32) and tile settings
(planner, 128 x 128, 256 x 256), with guard bands around every output and a non-zero
initial dW, against the float64 oracle.  The fused pass's dx must equal the x stage's bit
for bit (bf16, fp16)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import Guarded, device, note, oracle_b_chunked, oracle_w_chunked, oracle_x_rows
from parity import compare, forward_abs_models, sum_abs_model, to64
from workloads.gen import DTYPES, SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu


def _case(seed):
    rng = np.random.default_rng(90000 + seed)
    dt = ["bf16", "fp16", "fp32"][seed % 3]
    vec = 4 if dt == "fp32" else 8
    M = int(rng.integers(1, 6000)) if rng.random() < 0.8 else int(rng.integers(1, 40))
    K = (int(rng.integers(1, 1536 // vec + 1)) * vec if rng.random() < 0.85
         else vec * int(rng.integers(1, 4)))
    N = (int(rng.integers(1, 1536 // vec + 1)) * vec if rng.random() < 0.85
         else vec * int(rng.integers(1, 4)))
    tile = int(rng.choice([0, 128, 256]))
    return dt, M, K, N, tile


@pytest.mark.parametrize("seed", range(30))
def test_random_sweep(seed):
    dev = device()
    dt, M, K, N, tile = _case(seed)
    tdt = DTYPES[dt]
    note(f"random sweep {seed}: {dt} M={M} K={K} N={N} tile={tile}")
    inp = swiglu_inputs(SwiGLUShape("sweep", 700 + seed, M, K, N), dtype=dt)
    d = {k: v.to(dev) for k, v in inp.items()}
    swg.swg_set_gemm_tile(tile)
    try:
        # b stage
        dg, dfc = Guarded((M, N), tdt, dev), Guarded((M, N), tdt, dev)
        zero = torch.zeros(N, dtype=tdt, device=dev)
        db_g, db_fc = Guarded((N,), tdt, dev, fill=zero), Guarded((N,), tdt, dev, fill=zero)
        swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg.t, dfc.t, db_g.t, db_fc.t)
        torch.cuda.synchronize()
        for buf in (dg, dfc, db_g, db_fc):
            buf.check()
        res = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], gpu=(dg.t.cpu(), dfc.t.cpu()),
                               dtype=dt, store_dtype=tdt)
        res["check_dg"].result()
        res["check_dfc"].result()
        compare("db_g", db_g.t.cpu(), res["db_g"], dt, model_abs=sum_abs_model(res["abs_g"]),
                contraction=M)
        compare("db_fc", db_fc.t.cpu(), res["db_fc"], dt,
                model_abs=sum_abs_model(res["abs_fc"]), contraction=M)
        # w, x and the fused pass on the oracle's rounded dg / dfc, dW starting non-zero
        odg, odfc = res["dg"], res["dfc"]
        init = (torch.randn(K, N, generator=torch.Generator().manual_seed(seed)) * 0.01).to(tdt)
        i64 = to64(init)
        rg, rf, ag, af = oracle_w_chunked(inp["x"], odg, odfc)
        rx, ax = oracle_x_rows(odg, odfc, inp["w_g"], inp["w_fc"], slice(None))
        gdg, gdfc = odg.to(dev), odfc.to(dev)
        dx_sep = None
        for mode in ("separate", "fused"):
            dw_g = Guarded((K, N), tdt, dev, fill=init.to(dev))
            dw_fc = Guarded((K, N), tdt, dev, fill=init.to(dev))
            dx = Guarded((M, K), tdt, dev)
            if mode == "separate":
                swg.swiglu_bwd_w(d["x"], gdg, gdfc, dw_g.t, dw_fc.t)
                swg.swiglu_bwd_x(gdg, gdfc, d["w_g"], d["w_fc"], dx.t)
            else:
                swg.swiglu_bwd_wx(d["x"], gdg, gdfc, d["w_g"], d["w_fc"], dw_g.t, dw_fc.t, dx.t)
            torch.cuda.synchronize()
            for buf in (dw_g, dw_fc, dx):
                buf.check()
            compare(f"{mode} dw_g", dw_g.t.cpu(), rg + i64, dt,
                    model_abs=sum_abs_model(ag + np.abs(i64)), contraction=M)
            compare(f"{mode} dw_fc", dw_fc.t.cpu(), rf + i64, dt,
                    model_abs=sum_abs_model(af + np.abs(i64)), contraction=M)
            compare(f"{mode} dx", dx.t.cpu(), rx, dt, model_abs=sum_abs_model(ax),
                    contraction=2 * N)
            if mode == "separate":
                dx_sep = dx.t.clone()
            elif dt != "fp32":
                assert torch.equal(dx.t.view(torch.int16), dx_sep.view(torch.int16)), "fused dx"
        # forward
        g, fc, y = (Guarded((M, N), tdt, dev) for _ in range(3))
        swg.swiglu_fwd(d["x"], d["w_g"], d["w_fc"], d["b_g"], d["b_fc"], g.t, fc.t, y.t)
        torch.cuda.synchronize()
        for buf in (g, fc, y):
            buf.check()
        x64 = to64(inp["x"])
        fg, ff, fy = R.swiglu_forward_ref(x64, to64(inp["w_g"]), to64(inp["b_g"]),
                                          to64(inp["w_fc"]), to64(inp["b_fc"]))
        eg, ef, ey = forward_abs_models(x64, inp["w_g"], inp["w_fc"], inp["b_g"], inp["b_fc"],
                                        fg, ff)
        compare("g", g.t.cpu(), fg, dt, model_abs=eg, contraction=K)
        compare("fc", fc.t.cpu(), ff, dt, model_abs=ef, contraction=K)
        compare("y", y.t.cpu(), fy, dt, model_abs=ey, contraction=K)
    finally:
        swg.swg_set_gemm_tile(0)
