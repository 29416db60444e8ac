"""Kernel-duration timing (swg_time_next_call): a timed call dispatches its kernels with
the caller's events attached; its results must be bit-identical to an untimed call, the
events must span a positive time no longer than events recorded around the call, and the
setting must apply to one call only."""
from __future__ import annotations

import pytest
import torch

import swish_activation_backward_amd as swg
from gpu_util import device, note
from workloads.gen import swiglu_inputs

pytestmark = pytest.mark.gpu


def _events(stream, n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:           # torch creates the HIP event on its first record
        e.record(stream)
    torch.cuda.synchronize()
    return evs


def test_timed_calls_match_untimed_and_span_their_kernels():
    dev = device()
    inp = swiglu_inputs("ragged")
    d = {k: v.to(dev) for k, v in inp.items()}
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    bf = torch.bfloat16
    stream = torch.cuda.current_stream()

    def outs():
        return {"dg": torch.empty(M, N, dtype=bf, device=dev),
                "dfc": torch.empty(M, N, dtype=bf, device=dev),
                "db_g": torch.zeros(N, dtype=bf, device=dev),
                "db_fc": torch.zeros(N, dtype=bf, device=dev),
                "dw_g": torch.zeros(K, N, dtype=bf, device=dev),
                "dw_fc": torch.zeros(K, N, dtype=bf, device=dev),
                "dx": torch.empty(M, K, dtype=bf, device=dev),
                "gx": torch.empty(M, N, dtype=bf, device=dev)}

    def calls(o):
        return [
            ("b", lambda: swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], o["dg"], o["dfc"],
                                           o["db_g"], o["db_fc"])),
            ("w", lambda: swg.swiglu_bwd_w(d["x"], o["dg"], o["dfc"], o["dw_g"], o["dw_fc"])),
            ("x", lambda: swg.swiglu_bwd_x(o["dg"], o["dfc"], d["w_g"], d["w_fc"], o["dx"])),
            ("swish", lambda: swg.swish_grad(d["dy"], d["g"], grad_x=o["gx"], beta=1.702)),
        ]

    plain = outs()
    note("timing: untimed reference calls")
    for _, f in calls(plain):
        f()
    timed = outs()
    k = _events(stream, 8)
    br = _events(stream, 8)
    note("timing: timed calls")
    for i, (_, f) in enumerate(calls(timed)):
        br[2 * i].record(stream)
        swg.swg_time_next_call(k[2 * i], k[2 * i + 1])
        f()
        br[2 * i + 1].record(stream)
    # the setting was consumed: this call runs untimed and moves no event
    swg.swish_grad(d["dy"], d["g"], grad_x=timed["gx"], beta=1.702)
    torch.cuda.synchronize()
    for name in plain:
        assert torch.equal(plain[name].view(torch.int16), timed[name].view(torch.int16)), name
    for i, (name, _) in enumerate(calls(timed)):
        span = k[2 * i].elapsed_time(k[2 * i + 1])
        around = br[2 * i].elapsed_time(br[2 * i + 1])
        assert 0.0 < span <= around + 0.005, (name, span, around)


def test_time_next_call_needs_created_events():
    device()
    with pytest.raises(ValueError):
        swg.swg_time_next_call(torch.cuda.Event(enable_timing=True),
                               torch.cuda.Event(enable_timing=True))
    swg.swg_time_next_call(None, None)
