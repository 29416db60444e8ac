"""GPU parity at the full workload sizes, in the launch configuration the bench times:
the large-batch FFN shape (M=220000, K=512, N=1024) and the LLM-sized FFN
(M=16384, K=4096, N=14336), in bf16 and in fp16 (the Swish page lists fp16 beside bf16;
at the large-batch shape most fp16 dg / dfc values are fp16 subnormals, which the
checks' subnormal allowance covers).

Large-batch FFN: every output compared (the oracle runs over row blocks).
LLM FFN: dg, dfc and db in full; dw on 512 sampled columns of each of dw_g / dw_fc
(every row); dx on 1024 sampled rows plus the first and last rows.
The w and x stages are checked in isolation on the oracle's own dg / dfc rounded to
bf16, so no oracle input comes from the GPU path.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import device, note, oracle_b_chunked, oracle_w_chunked, oracle_x_rows
from parity import Checker, compare, sum_abs_model
from workloads.gen import DTYPES, swiglu_inputs

pytestmark = pytest.mark.gpu

_state = {}
CASES = [("ffn_220k", "bf16"), ("llm_ffn", "bf16"), ("ffn_220k", "fp16"), ("llm_ffn", "fp16")]


def _workload(name, dt):
    """Inputs, the GPU b-stage outputs and the oracle b stage (cached per workload)."""
    if _state.get("key") == (name, dt):
        return _state
    _state.clear()
    dev = device()
    tdt = DTYPES[dt]
    inp = swiglu_inputs(name, dtype=dt)
    M, N = inp["dy"].shape
    note(f"b stage {name} {dt} M={M} N={N}")
    d = {k: inp[k].to(dev) for k in ("dy", "g", "fc")}
    dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
    db_g = torch.zeros(N, dtype=tdt, device=dev)
    db_fc = torch.zeros_like(db_g)
    swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc)
    torch.cuda.synchronize()
    gpu = (dg.cpu(), dfc.cpu())
    del d, dg, dfc
    ref = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], gpu=gpu, store_dtype=tdt, dtype=dt)
    _state.update(key=(name, dt), inp=inp, ref=ref, db=(db_g.cpu(), db_fc.cpu()))
    return _state


@pytest.fixture(scope="module", params=CASES, ids=lambda c: f"{c[0]}-{c[1]}")
def case(request):
    """One workload and dtype; module scope makes pytest run every test of a case before
    the next case, so the large oracle b stage runs once per case."""
    return request.param


def test_full_b_stage(case):
    name, dt = case
    st = _workload(name, dt)
    ref = st["ref"]
    ref["check_dg"].result()
    ref["check_dfc"].result()
    compare("db_g", st["db"][0], ref["db_g"], dt, model_abs=sum_abs_model(ref["abs_g"]))
    compare("db_fc", st["db"][1], ref["db_fc"], dt, model_abs=sum_abs_model(ref["abs_fc"]))


def test_full_w_stage(case):
    name, dt = case
    st = _workload(name, dt)
    dev = device()
    inp, ref = st["inp"], st["ref"]
    M, K = inp["x"].shape
    N = inp["dy"].shape[1]
    dw_g = torch.zeros(K, N, dtype=DTYPES[dt], device=dev)
    dw_fc = torch.zeros_like(dw_g)
    note(f"w stage {name} {dt} M={M} K={K} N={N}")
    swg.swiglu_bwd_w(inp["x"].to(dev), ref["dg"].to(dev), ref["dfc"].to(dev), dw_g, dw_fc)
    torch.cuda.synchronize()
    cols = None
    if N > 4096:
        cols = np.sort(np.random.default_rng(17).choice(N, 512, replace=False))
    rg, rf, ag, af = oracle_w_chunked(inp["x"], ref["dg"], ref["dfc"], cols=cols)
    sel = slice(None) if cols is None else torch.from_numpy(cols)
    compare("dw_g", dw_g.cpu()[:, sel], rg, dt, model_abs=sum_abs_model(ag))
    compare("dw_fc", dw_fc.cpu()[:, sel], rf, dt, model_abs=sum_abs_model(af))


def test_full_x_stage(case):
    name, dt = case
    st = _workload(name, dt)
    dev = device()
    inp, ref = st["inp"], st["ref"]
    M, K = inp["x"].shape
    dx = torch.empty(M, K, dtype=DTYPES[dt], device=dev)
    note(f"x stage {name} {dt} M={M} K={K}")
    swg.swiglu_bwd_x(ref["dg"].to(dev), ref["dfc"].to(dev), inp["w_g"].to(dev),
                     inp["w_fc"].to(dev), dx)
    torch.cuda.synchronize()
    dx = dx.cpu()
    if M <= 250000 and K <= 1024:
        ck = Checker("dx", dt)
        for r0 in range(0, M, 32768):
            idx = slice(r0, min(M, r0 + 32768))
            r, a = oracle_x_rows(ref["dg"], ref["dfc"], inp["w_g"], inp["w_fc"], idx)
            ck.add(dx[idx], r, sum_abs_model(a))
        ck.result()
    else:
        rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(19).choice(M, 1024)]))
        idx = torch.from_numpy(rows)
        r, a = oracle_x_rows(ref["dg"], ref["dfc"], inp["w_g"], inp["w_fc"], idx)
        compare("dx", dx[idx], r, dt, model_abs=sum_abs_model(a))


def test_full_wx_fused(case):
    """The fused w + x pass in its bench configuration, on the oracle's rounded dg / dfc:
    dx bit-identical to the x stage's (whose parity is checked above, in full at the
    large-batch shape) and dW against the oracle (all columns at the large-batch shape,
    512 sampled columns at the LLM-sized FFN)."""
    name, dt = case
    st = _workload(name, dt)
    dev = device()
    inp, ref = st["inp"], st["ref"]
    M, K = inp["x"].shape
    N = inp["dy"].shape[1]
    tdt = DTYPES[dt]
    d = {"x": inp["x"].to(dev), "dg": ref["dg"].to(dev), "dfc": ref["dfc"].to(dev),
         "w_g": inp["w_g"].to(dev), "w_fc": inp["w_fc"].to(dev)}
    dw_g = torch.zeros(K, N, dtype=tdt, device=dev)
    dw_fc = torch.zeros_like(dw_g)
    dx = torch.empty(M, K, dtype=tdt, device=dev)
    note(f"fused w+x {name} {dt} M={M} K={K} N={N}")
    swg.swiglu_bwd_wx(d["x"], d["dg"], d["dfc"], d["w_g"], d["w_fc"], dw_g, dw_fc, dx)
    dx_sep = torch.empty_like(dx)
    swg.swiglu_bwd_x(d["dg"], d["dfc"], d["w_g"], d["w_fc"], dx_sep)
    torch.cuda.synchronize()
    assert torch.equal(dx.view(torch.int16), dx_sep.view(torch.int16)), "dx"
    del dx, dx_sep, d
    cols = None
    if N > 4096:
        cols = np.sort(np.random.default_rng(23).choice(N, 512, replace=False))
    rg, rf, ag, af = oracle_w_chunked(inp["x"], ref["dg"], ref["dfc"], cols=cols)
    sel = slice(None) if cols is None else torch.from_numpy(cols)
    compare("fused dw_g", dw_g.cpu()[:, sel], rg, dt, model_abs=sum_abs_model(ag))
    compare("fused dw_fc", dw_fc.cpu()[:, sel], rf, dt, model_abs=sum_abs_model(af))
