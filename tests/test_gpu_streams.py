"""Calls on a stream other than torch's current one: every binding takes ``stream=``; the
b and w stages then allocate their workspaces themselves and must keep them alive until
the kernels queued on that stream are done.  Results are compared bit for bit with the
same calls on the current stream (the kernels are deterministic)."""
from __future__ import annotations

import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import device, note
from workloads.gen import swiglu_inputs

pytestmark = pytest.mark.gpu


def _run(d, outs, stream, ws_bytes):
    dg, dfc, db_g, db_fc, dw_g, dw_fc, dx, gs, fs, ys, gx = outs
    dev = d["dy"].device
    swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc, stream=stream)
    # allocations of the workspaces' sizes on the current stream, written at once, while
    # the side stream may still run: they must not receive a workspace's memory
    junk = [torch.empty(n, dtype=torch.uint8, device=dev).fill_(0x7F) for n in ws_bytes]
    swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc, stream=stream)
    junk += [torch.empty(n, dtype=torch.uint8, device=dev).fill_(0x7F) for n in ws_bytes]
    swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx, stream=stream)
    swg.swiglu_fwd(d["x"], d["w_g"], d["w_fc"], d["b_g"], d["b_fc"], gs, fs, ys, stream=stream)
    swg.swish_grad(d["dy"], d["g"], grad_x=gx, beta=1.702, stream=stream)
    del junk


def test_side_stream_matches_current_stream():
    dev = device()
    inp = swiglu_inputs("ragged")
    d = {k: v.to(dev) for k, v in inp.items()}
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    bf = torch.bfloat16

    def outputs():
        return (torch.empty(M, N, dtype=bf, device=dev), torch.empty(M, N, dtype=bf, device=dev),
                torch.empty(N, dtype=bf, device=dev), torch.empty(N, dtype=bf, device=dev),
                torch.empty(K, N, dtype=bf, device=dev), torch.empty(K, N, dtype=bf, device=dev),
                torch.empty(M, K, dtype=bf, device=dev),
                *(torch.empty(M, N, dtype=bf, device=dev) for _ in range(3)),
                torch.empty(M, N, dtype=bf, device=dev))

    ws_bytes = [n for n in (swg.swiglu_bwd_b_workspace_size(M, N, bf),
                            swg.swiglu_bwd_w_workspace_size(M, K, N, bf)) if n > 0]
    assert ws_bytes, "the ragged workload should need a workspace"

    def zeroed():
        o = outputs()
        for t in o[2:6]:          # db_g, db_fc, dw_g, dw_fc accumulate
            t.zero_()
        return o

    note("streams: reference on the current stream")
    ref = zeroed()
    _run(d, ref, None, ws_bytes)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for rep in range(3):
        got = zeroed()
        s.wait_stream(torch.cuda.current_stream())   # inputs and zeroed outputs are ready
        note(f"streams: side stream, pass {rep}")
        _run(d, got, s, ws_bytes)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(got, ref)):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"output {i} differs"
