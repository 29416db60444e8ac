"""The static-scratch b stage (swiglu_bwd_b_noalloc, for callers that cannot allocate)
against swiglu_bwd_b with a caller workspace: bit-identical dg, dfc, db_g and db_fc on two
calls in a row, the second with a smaller input (fewer walkers, so fewer partial rows of
the shared array are read), each also checked against the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import device, note, oracle_b_chunked
from parity import compare, sum_abs_model, to64
from workloads.gen import SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu


def _run(entry, d, db0, dev):
    M, N = d["dy"].shape
    dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
    db_g, db_fc = db0.to(dev).clone(), (-db0).to(dev).clone()
    if entry == "noalloc":
        swg.swiglu_bwd_b_noalloc(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc)
    else:
        ws = torch.empty(max(1, swg.swiglu_bwd_b_workspace_size(M, N, d["dy"].dtype)),
                         dtype=torch.uint8, device=dev)
        swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc, workspace=ws)
    torch.cuda.synchronize()
    return [t.cpu() for t in (dg, dfc, db_g, db_fc)]


@pytest.mark.parametrize("dt", ["bf16"])
def test_noalloc_b_stage_matches_workspace_entry_point(dt):
    dev = device()
    shapes = [SwiGLUShape("noalloc_big", 31, 8191, 8, 1024),
              SwiGLUShape("noalloc_small", 32, 1000, 8, 264)]
    for shape in shapes:
        inp = swiglu_inputs(shape, dtype=dt)
        M, N = inp["dy"].shape
        d = {k: inp[k].to(dev) for k in ("dy", "g", "fc")}
        db0 = (torch.randn(N, generator=torch.Generator().manual_seed(shape.seed)) * 0.05
               ).to(inp["dy"].dtype)
        note(f"b stage noalloc vs workspace M={M} N={N} {dt}")
        got = _run("noalloc", d, db0, dev)
        want = _run("workspace", d, db0, dev)
        for name, a, b in zip(("dg", "dfc", "db_g", "db_fc"), got, want):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), name
        res = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], db0, -db0,
                               gpu=(got[0], got[1]), dtype=dt)
        res["check_dg"].result()
        res["check_dfc"].result()
        a0 = np.abs(to64(db0))
        compare("db_g", got[2], res["db_g"], dt, model_abs=sum_abs_model(res["abs_g"] + a0))
        compare("db_fc", got[3], res["db_fc"], dt, model_abs=sum_abs_model(res["abs_fc"] + a0))
