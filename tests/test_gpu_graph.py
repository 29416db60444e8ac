"""The backward path captured in a HIP graph (torch.cuda.CUDAGraph on ROCm): every library
call, the static-scratch b stage and the fused w + x pass included, is capturable (no
allocation, no memset nodes; accumulators are cleared with torch's fill kernel inside the
graph).  The graph is replayed several times with eager work and
synchronisations in between, and every replay is compared bit for bit with the eager run."""
from __future__ import annotations

import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import device, note
from workloads.gen import swiglu_inputs

pytestmark = pytest.mark.gpu


def test_backward_graph_replays_match_eager():
    dev = device()
    inp = swiglu_inputs("ragged")
    d = {k: v.to(dev) for k, v in inp.items()}
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    bf = torch.bfloat16
    dg, dfc = torch.empty(M, N, dtype=bf, device=dev), torch.empty(M, N, dtype=bf, device=dev)
    db_g, db_fc = torch.empty(N, dtype=bf, device=dev), torch.empty(N, dtype=bf, device=dev)
    dw_g, dw_fc = torch.empty(K, N, dtype=bf, device=dev), torch.empty(K, N, dtype=bf, device=dev)
    dx = torch.empty(M, K, dtype=bf, device=dev)
    gs, fs, ys = (torch.empty(M, N, dtype=bf, device=dev) for _ in range(3))
    gx = torch.empty_like(d["dy"])
    ws_b = torch.empty(max(1, swg.swiglu_bwd_b_workspace_size(M, N, bf)), dtype=torch.uint8,
                       device=dev)
    ws_w = torch.empty(max(1, swg.swiglu_bwd_w_workspace_size(M, K, N, bf)), dtype=torch.uint8,
                       device=dev)
    # the static-scratch b stage and the fused w + x pass into outputs of their own
    dg2, dfc2 = torch.empty_like(dg), torch.empty_like(dfc)
    db_g2, db_fc2 = torch.empty_like(db_g), torch.empty_like(db_fc)
    dw_g3, dw_fc3, dx3 = torch.empty_like(dw_g), torch.empty_like(dw_fc), torch.empty_like(dx)
    ws_wx = torch.empty(max(1, swg.swiglu_bwd_wx_workspace_size(M, K, N, bf)),
                        dtype=torch.uint8, device=dev)
    outs = (dg, dfc, db_g, db_fc, dw_g, dw_fc, dx, gs, fs, ys, gx, dg2, dfc2, db_g2, db_fc2,
            dw_g3, dw_fc3, dx3)
    names = ("dg", "dfc", "db_g", "db_fc", "dw_g", "dw_fc", "dx", "g", "fc", "y", "swish",
             "noalloc dg", "noalloc dfc", "noalloc db_g", "noalloc db_fc", "fused dw_g",
             "fused dw_fc", "fused dx")

    def step():
        for t in (db_g, db_fc, dw_g, dw_fc, db_g2, db_fc2, dw_g3, dw_fc3):
            t.zero_()
        swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc, workspace=ws_b)
        swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc, workspace=ws_w)
        swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx)
        swg.swiglu_fwd(d["x"], d["w_g"], d["w_fc"], d["b_g"], d["b_fc"], gs, fs, ys)
        swg.swish_grad(d["dy"], d["g"], grad_x=gx, beta=1.702)
        swg.swiglu_bwd_b_noalloc(d["dy"], d["g"], d["fc"], dg2, dfc2, db_g2, db_fc2)
        swg.swiglu_bwd_wx(d["x"], dg, dfc, d["w_g"], d["w_fc"], dw_g3, dw_fc3, dx3,
                          workspace=ws_wx)

    note("graph: eager reference")
    step()
    torch.cuda.synchronize()
    want = [t.view(torch.int16).clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    note("graph: capture")
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:            # eager work between replays: scribble over the outputs
            t.fill_(float(rep + 3))
        torch.cuda.synchronize()
        note(f"graph: replay {rep}")
        graph.replay()
        torch.cuda.synchronize()
        for name, t, w in zip(names, outs, want):
            assert torch.equal(t.view(torch.int16), w), f"replay {rep}: {name} differs"
    # the static-scratch b stage gives the workspace entry point's bits
    for a, b in ((dg2, dg), (dfc2, dfc), (db_g2, db_g), (db_fc2, db_fc), (dx3, dx)):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
