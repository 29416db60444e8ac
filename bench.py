#!/usr/bin/env python3
"""Throughput of the SwiGLU backward hot path on one MI355X.

One step = the three SwiGLU backward stages at the large-batch FFN shape of the Fused
SwiGLU backward page (M=220000 tokens, K=512, N=1024, bf16: b stage with the db column
sums, w-stage GEMM, x-stage GEMM) followed by the beta-scaled Swish gradient over
L = 2^24 + 37 elements in fp32, fp16 and bf16 (beta = 1.702).  Inputs are synthetic
(seeded), resident in HBM before timing starts.

Reported value: the step's fraction of its roofline, 100 * sum(roofline time of each
stage) / (measured step time), where a stage's roofline time is its algorithmic bytes
over 8 TB/s (HBM) or its flops over 2.5 PFLOP/s (dense bf16 MFMA), whichever is larger.
Each stage's absolute GB/s or TFLOP/s is listed too.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Defaults: 5 warm-up steps, 50 timed steps; per stage the mean (us), median, min and max
of the per-step kernel spans are reported.

Stage times are kernel spans: each library call is timed with swg_time_next_call, whose
HIP events are attached to the call's first and last kernel dispatch on the stream it
launches on (start of the first kernel to end of the last), the in-process equivalent of
a kernel trace.  Events recorded around each call are kept as `event_us` (they add the
dispatch gap, a few microseconds per call).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "SwiGLU-bwd GB/s (b kernel) + TFLOP/s (w/x GEMMs), % of roofline"
HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
MFMA_BF16_PEAK = 2.5e15    # flop/s, MI355X dense bf16 matrix cores
SWISH_BETA = 1.702
SWISH_DTYPES = ("fp32", "fp16", "bf16")
ES = {"fp32": 4, "fp16": 2, "bf16": 2}

# Kernel sources, hashed to tell whether recorded HBM counters still describe the code.
KERNEL_SOURCES = {
    "b_stage_kernel": "swish_activation_backward_amd/csrc/elementwise.hip",
    "w_stage_kernel": "swish_activation_backward_amd/csrc/gemm.hip",
    "x_stage_kernel": "swish_activation_backward_amd/csrc/gemm.hip",
    "swish_grad_vec_kernel": "swish_activation_backward_amd/csrc/elementwise.hip",
}

KERNELS = {
    "b": ["b_stage_kernel", "db_finalize_kernel"],
    "w": ["w_stage_kernel", "w_reduce_kernel"],
    "x": ["x_stage_kernel"],
    "swish_grad": ["swish_grad_vec_kernel"],
}


def stage_work(M, K, N, L):
    """Algorithmic bytes and flops per stage (extra traffic of partial sums excluded)."""
    w = {
        "b": {"bytes": 10 * M * N + 8 * N, "flops": 0},
        "w": {"bytes": 2 * M * K + 4 * M * N + 8 * K * N, "flops": 4 * M * K * N},
        "x": {"bytes": 4 * M * N + 4 * K * N + 2 * M * K, "flops": 4 * M * K * N},
    }
    for dt in SWISH_DTYPES:
        w[f"swish_grad_{dt}"] = {"bytes": 3 * ES[dt] * L, "flops": 0}
    for v in w.values():
        t_mem = v["bytes"] / HBM_PEAK
        t_mma = v["flops"] / MFMA_BF16_PEAK
        v["bound"] = "mfma" if t_mma > t_mem else "hbm"
        v["t_roof"] = max(t_mem, t_mma)
    return w


def source_sha256(rel):
    import hashlib
    with open(os.path.join(ROOT, rel), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def recorded_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary
    of this workload (scaled by the plain-copy calibration recorded with it), or None when
    there is no summary or the kernel's source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    try:
        with open(path) as f:
            text = f.read()
        block = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(block)["kernels"][kernel]
    except (OSError, IndexError, KeyError, ValueError):
        return None
    src = KERNEL_SOURCES.get(kernel)
    if src is None or rec.get("source_sha256") != source_sha256(src):
        return None
    return rec.get("hbm_bytes_per_launch")


class SpanTimer:
    """Pairs of torch events (created up front by one record each) handed to
    swg_time_next_call, so that a library call's kernels record them."""

    def __init__(self, swg, n):
        import torch
        self.swg = swg
        stream = torch.cuda.current_stream()
        self.ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)]
        for a, b in self.ev:
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()

    def arm(self, i):
        self.swg.swg_time_next_call(*self.ev[i])

    def seconds(self, i):
        a, b = self.ev[i]
        return a.elapsed_time(b) * 1e-3


def time_forward(swg, d, M, K, N, warmup, steps):
    """The SwiGLU forward entry point (g, fc, y from x, W, b) at the same shape, timed on
    its own after the step (it is not part of the backward step or of `value`)."""
    import torch
    g, fc, y = (torch.empty(M, N, dtype=torch.bfloat16, device=d["x"].device) for _ in range(3))
    args = (d["x"], d["w_g"], d["w_fc"], d["b_g"], d["b_fc"], g, fc, y)
    for _ in range(warmup):
        swg.swiglu_fwd(*args)
    timer = SpanTimer(swg, steps)
    for i in range(steps):
        timer.arm(i)
        swg.swiglu_fwd(*args)
    torch.cuda.synchronize()
    t = sum(timer.seconds(i) for i in range(steps)) / steps
    flops = 4.0 * M * K * N
    return {"us": round(t * 1e6, 2), "TFLOP/s": round(flops / t / 1e12, 1),
            "frac": round(flops / MFMA_BF16_PEAK / t, 4), "kernels": ["fwd_kernel"],
            "note": "SwiGLU forward (g, fc, y), mean kernel span, timed separately; not "
                    "part of the step"}


def time_fused(swg, d, dg, dfc, M, K, N, warmup, steps):
    """The fused w + x pass (swiglu_bwd_wx: dW and dx in one launch over [dg | dfc]) on the
    step's inputs, timed on its own beside the unfused w and x stages (not part of the
    step or of `value`).  Algorithmic work: the two GEMMs' flops; bytes x, [dg | dfc] and
    W read once, dx written, dW read and written."""
    import torch
    dev = d["x"].device
    dw_g = torch.zeros(K, N, dtype=torch.bfloat16, device=dev)
    dw_fc = torch.zeros_like(dw_g)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, swg.swiglu_bwd_wx_workspace_size(M, K, N, torch.bfloat16)),
                     dtype=torch.uint8, device=dev)
    args = (d["x"], dg, dfc, d["w_g"], d["w_fc"], dw_g, dw_fc, dx)
    for _ in range(warmup):
        swg.swiglu_bwd_wx(*args, workspace=ws)
    timer = SpanTimer(swg, steps)
    for i in range(steps):
        timer.arm(i)
        swg.swiglu_bwd_wx(*args, workspace=ws)
    torch.cuda.synchronize()
    ts = sorted(timer.seconds(i) for i in range(steps))
    t = sum(ts) / steps
    flops = 8.0 * M * K * N
    nbytes = 2 * M * K + 4 * M * N + 4 * K * N + 2 * M * K + 8 * K * N
    return {"us": round(t * 1e6, 2), "median_us": round(ts[len(ts) // 2] * 1e6, 2),
            "min_us": round(ts[0] * 1e6, 2), "TFLOP/s": round(flops / t / 1e12, 1),
            "GB/s": round(nbytes / t / 1e9, 1), "bound": "mfma",
            "frac": round(flops / MFMA_BF16_PEAK / t, 4),
            "kernels": ["wx_fused_kernel", "w_reduce_kernel"],
            "note": "fused w + x pass (swiglu_bwd_wx), mean kernel span on the step's "
                    "inputs; compare with stages w + x; not part of the step"}


def time_fp16(swg, d, M, K, N, warmup, steps):
    """The b, w and x stages on fp16 copies of the step's bf16 inputs (the same values
    rounded to fp16), each timed by its kernel span over `steps` calls after the step: the
    fp16 path at the headline shape, for comparison with the bf16 stages (not part of the
    step or of `value`; fp16 matrix cores have the bf16 peak)."""
    import torch
    h = {k: d[k].to(torch.float16) for k in ("x", "dy", "g", "fc", "w_g", "w_fc")}
    dg, dfc = torch.empty_like(h["dy"]), torch.empty_like(h["dy"])
    db_g = torch.zeros(N, dtype=torch.float16, device=h["x"].device)
    db_fc = torch.zeros_like(db_g)
    dw_g = torch.zeros(K, N, dtype=torch.float16, device=h["x"].device)
    dw_fc = torch.zeros_like(dw_g)
    dx = torch.empty(M, K, dtype=torch.float16, device=h["x"].device)
    ws_b = torch.empty(max(1, swg.swiglu_bwd_b_workspace_size(M, N, torch.float16)),
                       dtype=torch.uint8, device=h["x"].device)
    ws_w = torch.empty(max(1, swg.swiglu_bwd_w_workspace_size(M, K, N, torch.float16)),
                       dtype=torch.uint8, device=h["x"].device)
    calls = {
        "b": lambda: swg.swiglu_bwd_b(h["dy"], h["g"], h["fc"], dg, dfc, db_g, db_fc,
                                      workspace=ws_b),
        "w": lambda: swg.swiglu_bwd_w(h["x"], dg, dfc, dw_g, dw_fc, workspace=ws_w),
        "x": lambda: swg.swiglu_bwd_x(dg, dfc, h["w_g"], h["w_fc"], dx),
    }
    work = stage_work(M, K, N, 0)
    out = {"note": "b, w, x on fp16 copies of the step's inputs, mean kernel span; not part "
                   "of the step"}
    for name, f in calls.items():
        for _ in range(warmup):
            f()
        timer = SpanTimer(swg, steps)
        for i in range(steps):
            timer.arm(i)
            f()
        torch.cuda.synchronize()
        t = sum(timer.seconds(i) for i in range(steps)) / steps
        wk = work[name]
        e = {"us": round(t * 1e6, 2), "frac": round(wk["t_roof"] / t, 4), "bound": wk["bound"]}
        if wk["flops"]:
            e["TFLOP/s"] = round(wk["flops"] / t / 1e12, 1)
        else:
            e["GB/s"] = round(wk["bytes"] / t / 1e9, 1)
        out[name] = e
    del h, dg, dfc, dx, dw_g, dw_fc, ws_b, ws_w
    torch.cuda.empty_cache()
    return out


class Evictor:
    """Evicts the 256 MB last-level cache before a cold timed call by reading a 1 GiB
    buffer (a read-only pass: the timed call then finds its inputs in HBM and no dirty
    lines of an unrelated kernel left to write back)."""

    def __init__(self, dev):
        import torch
        # float32: torch sums it in place (an int32 sum would first cast to int64, a
        # 2 GiB write)
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.sum()


def time_swish_context(swg, steps):
    """The Swish gradient on the one workload the pages time: an fp16 [32, 64, 56, 56]
    activation with beta = 1 (Ascend C custom-operator page, performance table).  Each
    call is preceded by a 1 GiB read (Evictor), so its inputs come from HBM and not from
    the 256 MB last-level cache; each call is timed by its kernel span.  Reported beside
    the step, not part of `value`."""
    import torch
    from workloads.gen import SWISH_CONTEXT, swish_inputs
    c = SWISH_CONTEXT
    L = 1
    for s in c["shape"]:
        L *= s
    dev = torch.device("cuda", 0)
    inp = {k: v.reshape(c["shape"]).to(dev) for k, v in
           swish_inputs(c["dtype"], L=L, seed=c["seed"]).items()}
    out = torch.empty_like(inp["grad"])
    evict = Evictor(dev)
    timer = SpanTimer(swg, steps + 3)
    times = []
    for i in range(steps + 3):
        evict()
        timer.arm(i)
        swg.swish_grad(inp["grad"], inp["x"], grad_x=out, beta=c["beta"])
        torch.cuda.synchronize()
        if i >= 3:
            times.append(timer.seconds(i))
    times.sort()
    t = times[len(times) // 2]
    nbytes = 3 * 2 * L
    return {"shape": list(c["shape"]), "dtype": c["dtype"], "beta": c["beta"],
            "median_us": round(t * 1e6, 2), "min_us": round(times[0] * 1e6, 2),
            "GB/s": round(nbytes / t / 1e9, 1), "frac": round(nbytes / HBM_PEAK / t, 4),
            "pages_us": {"ascend_c_kernel": 280, "autodiff": 420},
            "note": "median kernel span of one call after a 1 GiB cache-evicting read; "
                    "the pages' times are Ascend 910B, context only"}


def time_configs(swg, names=("tiny", "ragged", "llm_ffn"), warmup=3, steps=10):
    """The b, w and x stages and the fused w + x pass at the other SwiGLU workloads (same
    seeded recipe), each
    stage call preceded by a 1 GiB read that evicts the 256 MB last-level cache (the
    tiny and ragged working sets would otherwise stay in it; a read leaves no dirty lines
    for the timed call to write back) and timed by its kernel span, median over `steps`
    calls.  Reported beside the step (the tiny and ragged
    shapes are launch- and latency-bound; the LLM-sized FFN is matrix-core bound); not
    part of `value`."""
    import torch
    from workloads.gen import SWIGLU_WORKLOADS, swiglu_inputs
    dev = torch.device("cuda", 0)
    evict = Evictor(dev)
    res = {}
    for name in names:
        shape = SWIGLU_WORKLOADS[name]
        M, K, N = shape.M, shape.K, shape.N
        d = {k: v.to(dev) for k, v in swiglu_inputs(shape).items()}
        dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
        db_g = torch.zeros(N, dtype=torch.bfloat16, device=dev)
        db_fc = torch.zeros_like(db_g)
        dw_g = torch.zeros(K, N, dtype=torch.bfloat16, device=dev)
        dw_fc = torch.zeros_like(dw_g)
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        ws_b = torch.empty(max(1, swg.swiglu_bwd_b_workspace_size(M, N, torch.bfloat16)),
                           dtype=torch.uint8, device=dev)
        ws_w = torch.empty(max(1, swg.swiglu_bwd_w_workspace_size(M, K, N, torch.bfloat16)),
                           dtype=torch.uint8, device=dev)
        ws_wx = torch.empty(max(1, swg.swiglu_bwd_wx_workspace_size(M, K, N, torch.bfloat16)),
                            dtype=torch.uint8, device=dev)
        calls = {
            "b": lambda: swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc,
                                          workspace=ws_b),
            "w": lambda: swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc, workspace=ws_w),
            "x": lambda: swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx),
            "fused_wx": lambda: swg.swiglu_bwd_wx(d["x"], dg, dfc, d["w_g"], d["w_fc"], dw_g,
                                                  dw_fc, dx, workspace=ws_wx),
        }
        for _ in range(warmup):
            for f in calls.values():
                f()
        timer = SpanTimer(swg, steps * len(calls))
        for it in range(steps):
            for i, f in enumerate(calls.values()):
                evict()
                timer.arm(it * len(calls) + i)
                f()
        torch.cuda.synchronize()
        work = stage_work(M, K, N, 0)
        work["fused_wx"] = {"flops": work["w"]["flops"] + work["x"]["flops"],
                            "t_roof": work["w"]["t_roof"] + work["x"]["t_roof"],
                            "bound": work["w"]["bound"]}
        out = {"M": M, "K": K, "N": N}
        for i, st in enumerate(calls):
            ts = sorted(timer.seconds(it * len(calls) + i) for it in range(steps))
            t = ts[len(ts) // 2]
            wk = work[st]
            e = {"median_us": round(t * 1e6, 2), "frac": round(wk["t_roof"] / t, 4),
                 "bound": wk["bound"]}
            if wk["flops"]:
                e["TFLOP/s"] = round(wk["flops"] / t / 1e12, 1)
            else:
                e["GB/s"] = round(wk["bytes"] / t / 1e9, 1)
            out[st] = e
        res[name] = out
        del calls, d, dg, dfc, dx, dw_g, dw_fc, ws_b, ws_w, ws_wx
        torch.cuda.empty_cache()
    return res


def measured_copy_rate(reps=10, nbytes=1 << 30):
    """HBM rate of a plain device-to-device copy (torch copy_, 1 GiB read + 1 GiB written),
    the practical ceiling the HBM-bound stages are also compared with (context only: the
    roofline peak stays the 8 TB/s specification)."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(2):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    e1.synchronize()
    t = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2.0 * nbytes / t


def copy_calibration(nbytes, reps=5):
    """A plain device-to-device copy of `nbytes`, for scaling the HBM byte counters."""
    import torch
    dev = torch.device("cuda", 0)
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "launches": reps}), flush=True)


def cpu_baseline(inp, sw_inputs, rows, swish_len):
    """The float64 oracle, as it stands, on a bounded sample of the same workload."""
    import oracle.ref as R
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()
                            if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        blas_threads = len(os.sched_getaffinity(0))
    f64 = lambda t: t.double().numpy()  # noqa: E731
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    m = min(rows, M)
    dy, g, fc, x = (f64(inp[k][:m]) for k in ("dy", "g", "fc", "x"))
    wg, wf = f64(inp["w_g"]), f64(inp["w_fc"])
    swish_len = min(swish_len, sw_inputs["fp32"]["grad"].numel())
    sw = {dt: (f64(v["grad"][:swish_len]), f64(v["x"][:swish_len])) for dt, v in sw_inputs.items()}
    stages = {}

    def timed(name, fn):
        """Run one oracle stage; record its wall seconds and the cores it kept busy
        (process CPU time over wall time, all threads of the process)."""
        w0, c0 = time.perf_counter(), time.process_time()
        out = fn()
        w, c = time.perf_counter() - w0, time.process_time() - c0
        stages[name] = {"seconds": round(w, 4), "cores_used": round(c / w, 2) if w > 0 else None}
        return out

    # the element-wise stages run before the matmuls: BLAS worker threads spin for a while
    # after a matmul, which would be counted against the stage that follows it
    t0 = time.perf_counter()
    dg, dfc, _, _ = timed("b", lambda: R.b_ref(dy, g, fc))
    for dt in SWISH_DTYPES:
        timed(f"swish_grad_{dt}", lambda dt=dt: R.swish_grad_ref(sw[dt][0], sw[dt][1], SWISH_BETA))
    timed("w", lambda: R.w_ref(x, dg, dfc))
    timed("x", lambda: R.x_ref(dg, dfc, wg, wf))
    t = time.perf_counter() - t0
    work = stage_work(m, K, N, swish_len)
    t_roof = sum(v["t_roof"] for v in work.values())
    used = max(v["cores_used"] or 0 for v in stages.values())
    return {"value": round(100.0 * t_roof / t, 6), "unit": "% of roofline",
            "cores": max(1, int(round(used))), "kind": "oracle",
            "seconds": round(t, 3), "stages": stages,
            "blas": _blas_info(), "host_cores": len(os.sched_getaffinity(0)),
            "blas_threads": int(blas_threads),
            "sample": f"{m} of {M} rows (b, w, x stages) and {swish_len} elements of the "
                      f"Swish input per dtype (whole workload when equal); numpy float64; "
                      f"cores = the most any stage kept busy (stages.*.cores_used: process "
                      f"CPU time / wall time; numpy element-wise stages run on one thread, "
                      f"the w and x matmuls on the BLAS threads)",
            "cpu": _cpu_model()}


def _blas_info():
    """The BLAS library numpy calls (threadpoolctl), e.g. 'openblas 0.3.x'."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
    except Exception:  # pragma: no cover
        pass
    return "unknown"


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="ffn_220k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true",
                    help="skip timing the b, w and x stages at the other SwiGLU workloads")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of BYTES bytes (counter calibration) and exit")
    ap.add_argument("--cpu-rows", type=int, default=1 << 30,
                    help="rows of the SwiGLU workload the oracle baseline runs (default: all "
                         "of them; a few seconds of float64 work on a 16-core host)")
    ap.add_argument("--cpu-swish-len", type=int, default=1 << 30,
                    help="Swish elements per dtype for the oracle baseline (default: all)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the data-parallel "
              "split over M and its all-reduce of db/dw are design notes only); run with "
              "--gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration > 0:
        copy_calibration(args.copy_calibration)
        return

    import swish_activation_backward_amd as swg
    from workloads.gen import SWIGLU_WORKLOADS, SWISH_WORKLOAD, swiglu_inputs, swish_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    swg.load_library()
    dev = torch.device("cuda", 0)
    shape = SWIGLU_WORKLOADS[args.workload]
    M, K, N = shape.M, shape.K, shape.N
    L = SWISH_WORKLOAD["L"]

    inp = swiglu_inputs(shape)
    sw_inputs = {dt: swish_inputs(dt) for dt in SWISH_DTYPES}
    d = {k: v.to(dev) for k, v in inp.items()}
    sw = {dt: {k: v.to(dev) for k, v in s.items()} for dt, s in sw_inputs.items()}
    sw_out = {dt: torch.empty_like(sw[dt]["grad"]) for dt in SWISH_DTYPES}
    dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
    db_g = torch.zeros(N, dtype=torch.bfloat16, device=dev)
    db_fc = torch.zeros_like(db_g)
    dw_g = torch.zeros(K, N, dtype=torch.bfloat16, device=dev)
    dw_fc = torch.zeros_like(dw_g)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    ws_b = torch.empty(max(1, swg.swiglu_bwd_b_workspace_size(M, N, torch.bfloat16)),
                       dtype=torch.uint8, device=dev)
    ws_w = torch.empty(max(1, swg.swiglu_bwd_w_workspace_size(M, K, N, torch.bfloat16)),
                       dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    calls = [
        ("b", lambda: swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc,
                                       workspace=ws_b)),
        ("w", lambda: swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc, workspace=ws_w)),
        ("x", lambda: swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx)),
    ] + [(f"swish_grad_{dt}",
          (lambda dt=dt: swg.swish_grad(sw[dt]["grad"], sw[dt]["x"], grad_x=sw_out[dt],
                                        beta=SWISH_BETA)))
         for dt in SWISH_DTYPES]
    names = [n for n, _ in calls]

    def step(s=None):
        for i, (_, f) in enumerate(calls):
            if s is not None:
                events[s][i].record(stream)
                spans.arm(s * len(calls) + i)
            f()
        if s is not None:
            events[s][len(calls)].record(stream)

    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
              for _ in range(args.steps)]
    spans = SpanTimer(swg, args.steps * len(calls))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    samples = {n: [spans.seconds(s * len(calls) + i) for s in range(args.steps)]
               for i, n in enumerate(names)}
    around = {n: [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for ev in events]
              for i, n in enumerate(names)}
    per_stage = {n: sum(v) / len(v) for n, v in samples.items()}
    step_s = sum(per_stage.values())
    event_step_s = sum(sum(v) / len(v) for v in around.values())
    work = stage_work(M, K, N, L)
    t_roof = sum(v["t_roof"] for v in work.values())

    stages = {}
    for n in names:
        t = per_stage[n]
        wk = work[n]
        srt = sorted(samples[n])
        e = {"us": round(t * 1e6, 2),
             "median_us": round(srt[len(srt) // 2] * 1e6, 2),
             "min_us": round(srt[0] * 1e6, 2), "max_us": round(srt[-1] * 1e6, 2),
             "event_us": round(sum(around[n]) / len(around[n]) * 1e6, 2),
             "GB/s": round(wk["bytes"] / t / 1e9, 1),
             "bound": wk["bound"], "roofline_us": round(wk["t_roof"] * 1e6, 2),
             "frac": round(wk["t_roof"] / t, 4),
             "kernels": KERNELS["swish_grad" if n.startswith("swish") else n]}
        if wk["flops"]:
            e["TFLOP/s"] = round(wk["flops"] / t / 1e12, 1)
        stages[n] = e
    dom = max(names, key=lambda n: per_stage[n])
    wk, t = work[dom], per_stage[dom]
    if wk["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": round(wk["flops"] / t / 1e12, 2),
                "peak": MFMA_BF16_PEAK / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(wk["bytes"] / t / 1e9, 1),
                "peak": HBM_PEAK / 1e9, "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = recorded_traffic(args.workload, stages[dom]["kernels"][0])
    roof["stage"] = dom
    roof["kernels"] = stages[dom]["kernels"]
    roof["avg_launch_us"] = stages[dom]["us"]

    out = {
        "metric": METRIC,
        "value": round(100.0 * t_roof / step_s, 3),
        "unit": "% of roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"swiglu_bwd {shape.name} M={M} K={K} N={N} bf16 + swish_grad "
                               f"L={L} fp32/fp16/bf16 beta={SWISH_BETA}",
                   "M": M, "K": K, "N": N, "swish_L": L, "parallelism": "single GPU"},
        "kernel_ms_per_step": round(step_s * 1e3, 4),
        "event_ms_per_step": round(event_step_s * 1e3, 4),
        "timing": "stage us = mean kernel span per call (HIP events attached to the call's "
                  "first and last kernel dispatch with swg_time_next_call); event_us = events "
                  "recorded around the call; value = 100 * roofline time / kernel time",
        "roofline_ms_per_step": round(t_roof * 1e3, 4),
        "stages": stages,
        "roofline": roof,
    }
    copy_rate = measured_copy_rate()
    out["hbm_copy"] = {"GB/s": round(copy_rate / 1e9, 1),
                       "note": "plain 1 GiB device-to-device copy (torch copy_), read + write bytes"}
    for n in names:
        if stages[n]["bound"] == "hbm":
            stages[n]["frac_of_copy"] = round(work[n]["bytes"] / per_stage[n] / copy_rate, 4)
    out["fused_wx"] = time_fused(swg, d, dg, dfc, M, K, N, args.warmup, args.steps)
    out["fused_wx"]["unfused_w_plus_x_us"] = round(stages["w"]["us"] + stages["x"]["us"], 2)
    out["forward"] = time_forward(swg, d, M, K, N, args.warmup, args.steps)
    out["fp16"] = time_fp16(swg, d, M, K, N, args.warmup, args.steps)
    out["swish_pages_shape"] = time_swish_context(swg, 20)
    if not args.no_per_config:
        out["per_config"] = time_configs(swg)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, sw_inputs, args.cpu_rows, args.cpu_swish_len)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
