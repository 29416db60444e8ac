"""GPU parity of the SwiGLU backward stages (through the C ABI) against the float64 oracle:
the tiny and ragged-batch workloads in full, odd shapes, accumulation into non-zero
buffers, the chained b -> w -> x path, determinism and guard bands."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import Guarded, device, note, oracle_b_chunked, oracle_w_chunked, oracle_x_rows, rne
from parity import (Checker, chained_abs_model, compare, dfc_abs_model, dg_abs_model,
                    sum_abs_model, to64)
from workloads.gen import DTYPES, SwiGLUShape, swiglu_inputs

pytestmark = pytest.mark.gpu


def _b_case(inp, dt, db0=None):
    dev = device()
    M, N = inp["dy"].shape
    tdt = DTYPES[dt]
    dy, g, fc = (inp[k].to(dev) for k in ("dy", "g", "fc"))
    dg, dfc = Guarded((M, N), tdt, dev), Guarded((M, N), tdt, dev)
    init = torch.zeros(N, dtype=tdt) if db0 is None else db0
    db_g, db_fc = Guarded((N,), tdt, dev, fill=init.to(dev)), Guarded((N,), tdt, dev, fill=(-init).to(dev))
    note(f"b stage M={M} N={N} {dt} init={'zero' if db0 is None else 'nonzero'}")
    swg.swiglu_bwd_b(dy, g, fc, dg.t, dfc.t, db_g.t, db_fc.t)
    torch.cuda.synchronize()
    for buf in (dg, dfc, db_g, db_fc):
        buf.check()
    res = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], init, -init,
                           gpu=(dg.t.cpu(), dfc.t.cpu()), dtype=dt)
    res["check_dg"].result()
    res["check_dfc"].result()
    compare("db_g", db_g.t.cpu(), res["db_g"], dt,
            model_abs=sum_abs_model(res["abs_g"] + np.abs(to64(init))), contraction=M)
    compare("db_fc", db_fc.t.cpu(), res["db_fc"], dt,
            model_abs=sum_abs_model(res["abs_fc"] + np.abs(to64(init))), contraction=M)
    return dg.t, dfc.t


def _w_case(x, dg, dfc, dt, dw0=None):
    dev = device()
    M, K = x.shape
    N = dg.shape[1]
    tdt = DTYPES[dt]
    init = torch.zeros(K, N, dtype=tdt) if dw0 is None else dw0
    dw_g = Guarded((K, N), tdt, dev, fill=init.to(dev))
    dw_fc = Guarded((K, N), tdt, dev, fill=(2 * init).to(dev))
    note(f"w stage M={M} K={K} N={N} {dt} init={'zero' if dw0 is None else 'nonzero'}")
    swg.swiglu_bwd_w(x.to(dev), dg.to(dev), dfc.to(dev), dw_g.t, dw_fc.t)
    torch.cuda.synchronize()
    dw_g.check()
    dw_fc.check()
    rg, rf, ag, af = oracle_w_chunked(x, dg, dfc)
    i64 = to64(init)
    compare("dw_g", dw_g.t.cpu(), rg + i64, dt, model_abs=sum_abs_model(ag + np.abs(i64)),
            contraction=M)
    compare("dw_fc", dw_fc.t.cpu(), rf + 2 * i64, dt,
            model_abs=sum_abs_model(af + 2 * np.abs(i64)), contraction=M)
    return dw_g.t, dw_fc.t


def _x_case(dg, dfc, w_g, w_fc, dt):
    dev = device()
    M, N = dg.shape
    K = w_g.shape[0]
    dx = Guarded((M, K), DTYPES[dt], dev)
    note(f"x stage M={M} K={K} N={N} {dt}")
    swg.swiglu_bwd_x(dg.to(dev), dfc.to(dev), w_g.to(dev), w_fc.to(dev), dx.t)
    torch.cuda.synchronize()
    dx.check()
    ref, a = oracle_x_rows(dg, dfc, w_g, w_fc, slice(None))
    compare("dx", dx.t.cpu(), ref, dt, model_abs=sum_abs_model(a), contraction=2 * N)
    return dx.t


def _oracle_dg(inp, dt):
    res = oracle_b_chunked(inp["dy"], inp["g"], inp["fc"], store_dtype=DTYPES[dt])
    return res["dg"], res["dfc"]


@pytest.mark.parametrize("wl", ["tiny", "ragged"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_b_stage_workloads(wl, dt):
    inp = swiglu_inputs(wl, dtype=dt)
    _b_case(inp, dt)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_b_stage_accumulates_into_nonzero_db(dt):
    inp = swiglu_inputs("ragged", dtype=dt)
    N = inp["dy"].shape[1]
    db0 = (torch.randn(N, generator=torch.Generator().manual_seed(5)) * 0.05).to(DTYPES[dt])
    _b_case(inp, dt, db0=db0)


@pytest.mark.parametrize("M,N", [(1, 1), (37, 13), (300, 8), (129, 1000), (2, 2056),
                                 (4097, 24), (5, 4104), (70000, 16), (3001, 200),
                                 (20000, 120)])
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_b_stage_odd_shapes(M, N, dt):
    inp = swiglu_inputs(SwiGLUShape("odd", 11, M, 8, N), dtype=dt)
    _b_case(inp, dt)


def test_b_stage_unaligned_rows_use_scalar_path():
    """N = 12: rows are not 16-byte aligned, so the element-wise path runs."""
    inp = swiglu_inputs(SwiGLUShape("odd", 12, 999, 8, 12), dtype="bf16")
    _b_case(inp, "bf16")


@pytest.mark.parametrize("wl", ["tiny", "ragged"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_w_stage_workloads(wl, dt, tile):
    inp = swiglu_inputs(wl, dtype=dt)
    dg, dfc = _oracle_dg(inp, dt)
    _w_case(inp["x"], dg, dfc, dt)


def test_w_stage_accumulates_into_nonzero_dw(tile):
    inp = swiglu_inputs("ragged", dtype="bf16")
    dg, dfc = _oracle_dg(inp, "bf16")
    K, N = inp["w_g"].shape
    dw0 = (torch.randn(K, N, generator=torch.Generator().manual_seed(8)) * 1e-3).to(torch.bfloat16)
    _w_case(inp["x"], dg, dfc, "bf16", dw0=dw0)


@pytest.mark.parametrize("wl", ["tiny", "ragged"])
@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_x_stage_workloads(wl, dt, tile):
    inp = swiglu_inputs(wl, dtype=dt)
    dg, dfc = _oracle_dg(inp, dt)
    _x_case(dg, dfc, inp["w_g"], inp["w_fc"], dt)


@pytest.mark.parametrize("M,K,N", [(1, 8, 8), (63, 72, 136), (300, 264, 264), (1000, 8, 520),
                                   (257, 520, 8), (700, 256, 128), (513, 1032, 72),
                                   (2000, 64, 2048), (300, 200, 64), (129, 96, 192)])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_gemm_stages_odd_shapes(M, K, N, dt, tile):
    inp = swiglu_inputs(SwiGLUShape("odd", 13, M, K, N), dtype=dt)
    dg, dfc = _oracle_dg(inp, dt)
    _w_case(inp["x"], dg, dfc, dt)
    _x_case(dg, dfc, inp["w_g"], inp["w_fc"], dt)


@pytest.mark.parametrize("M,K,N", [(1, 4, 4), (63, 36, 132), (300, 260, 268), (129, 96, 196),
                                   (700, 256, 128), (2000, 4, 1028), (513, 1028, 76),
                                   (2211, 896, 1504)])
def test_gemm_stages_fp32_odd_shapes(M, K, N):
    """The fp32 path: K and N multiples of 4, partial tiles on every side, M split or not;
    the last shape's x stage sums 3008 products per output (the fp32 normwise bound then
    follows the contraction length)."""
    inp = swiglu_inputs(SwiGLUShape("odd32", 14, M, K, N), dtype="fp32")
    dg, dfc = _oracle_dg(inp, "fp32")
    _w_case(inp["x"], dg, dfc, "fp32")
    _x_case(dg, dfc, inp["w_g"], inp["w_fc"], "fp32")


@pytest.mark.parametrize("M,K,N", [(8191, 512, 1024), (300, 264, 264), (2000, 64, 2048),
                                   (513, 1032, 72), (20000, 520, 1000)])
@pytest.mark.parametrize("dt", ["bf16", "fp16"])
def test_x_stage_bits_do_not_depend_on_tile(M, K, N, dt):
    """Every dx element sees the same matrix-core operations in the same contraction order
    at either tile size, so the two configurations give the same bits."""
    dev = device()
    inp = swiglu_inputs(SwiGLUShape("xtile", 15, M, K, N), dtype=dt)
    d = {k: inp[k].to(dev) for k in ("dy", "w_g", "w_fc")}
    out = {}
    for edge in (128, 256):
        note(f"x stage tile {edge} M={M} K={K} N={N} {dt}")
        swg.swg_set_gemm_tile(edge)
        try:
            dx = torch.empty(M, K, dtype=DTYPES[dt], device=dev)
            swg.swiglu_bwd_x(d["dy"], d["dy"], d["w_g"], d["w_fc"], dx)
            torch.cuda.synchronize()
            out[edge] = dx.cpu()
        finally:
            swg.swg_set_gemm_tile(0)
    assert torch.equal(out[128].view(torch.int16), out[256].view(torch.int16))


def _random_shape(seed, vec):
    """A seeded shape with K, N multiples of `vec` (the 16-byte row rule), sizes spread
    over several tiles and partial tiles on every side."""
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.integers(1, 3000))
    K = int(rng.integers(1, 1100 // vec + 1)) * vec
    N = int(rng.integers(1, 1100 // vec + 1)) * vec
    return M, K, N


@pytest.mark.parametrize("seed", range(12))
def test_gemm_stages_random_shapes(seed, tile):
    """Seeded random shapes (bf16 and fp16 alternately): w and x against the oracle."""
    M, K, N = _random_shape(seed, 8)
    dt = "bf16" if seed % 2 == 0 else "fp16"
    inp = swiglu_inputs(SwiGLUShape("rand", 40 + seed, M, K, N), dtype=dt)
    dg, dfc = _oracle_dg(inp, dt)
    _w_case(inp["x"], dg, dfc, dt)
    _x_case(dg, dfc, inp["w_g"], inp["w_fc"], dt)


@pytest.mark.parametrize("seed", range(6))
def test_gemm_stages_large_random_shapes(seed, tile):
    """Seeded larger shapes (M up to 60000, K and N up to 4096, ragged edges) at both tile
    sizes: w on 96 sampled columns of dW, x on 192 sampled rows of dx, against the oracle."""
    rng = np.random.default_rng(5000 + seed)
    M = int(rng.integers(1000, 60000))
    K = int(rng.integers(1, 4096 // 8 + 1)) * 8
    N = int(rng.integers(1, 4096 // 8 + 1)) * 8
    dt = "bf16" if seed % 2 == 0 else "fp16"
    dev = device()
    tdt = DTYPES[dt]
    g = torch.Generator().manual_seed(6000 + seed)
    r = lambda *s, sc: (torch.randn(*s, generator=g) * sc).to(tdt)  # noqa: E731
    x, dg, dfc = r(M, K, sc=M ** -0.5), r(M, N, sc=1e-2), r(M, N, sc=1e-2)
    w_g, w_fc = r(K, N, sc=K ** -0.5), r(K, N, sc=K ** -0.5)
    note(f"large random gemm M={M} K={K} N={N} {dt} tile {tile}")
    dw_g, dw_fc = Guarded((K, N), tdt, dev, fill=torch.zeros(K, N, dtype=tdt, device=dev)), \
        Guarded((K, N), tdt, dev, fill=torch.zeros(K, N, dtype=tdt, device=dev))
    dx = Guarded((M, K), tdt, dev)
    d = {k: v.to(dev) for k, v in (("x", x), ("dg", dg), ("dfc", dfc), ("w_g", w_g), ("w_fc", w_fc))}
    swg.swiglu_bwd_w(d["x"], d["dg"], d["dfc"], dw_g.t, dw_fc.t)
    swg.swiglu_bwd_x(d["dg"], d["dfc"], d["w_g"], d["w_fc"], dx.t)
    torch.cuda.synchronize()
    for buf in (dw_g, dw_fc, dx):
        buf.check()
    cols = np.sort(rng.choice(N, min(N, 96), replace=False))
    rows = np.sort(rng.choice(M, min(M, 192), replace=False))
    rg, rf, ag, af = oracle_w_chunked(x, dg, dfc, cols=cols)
    compare("dw_g cols", dw_g.t.cpu()[:, cols], rg, dt, model_abs=sum_abs_model(ag))
    compare("dw_fc cols", dw_fc.t.cpu()[:, cols], rf, dt, model_abs=sum_abs_model(af))
    ref, a = oracle_x_rows(dg, dfc, w_g, w_fc, rows)
    compare("dx rows", dx.t.cpu()[rows], ref, dt, model_abs=sum_abs_model(a))


@pytest.mark.parametrize("seed", range(6))
def test_gemm_stages_fp32_random_shapes(seed):
    M, K, N = _random_shape(100 + seed, 4)
    inp = swiglu_inputs(SwiGLUShape("rand32", 60 + seed, M, K, N), dtype="fp32")
    dg, dfc = _oracle_dg(inp, "fp32")
    _w_case(inp["x"], dg, dfc, "fp32")
    _x_case(dg, dfc, inp["w_g"], inp["w_fc"], "fp32")


def test_w_stage_fp32_accumulates_into_nonzero_dw():
    """Split partials (M = 8191) added to a non-zero fp32 dw."""
    inp = swiglu_inputs("ragged", dtype="fp32")
    dg, dfc = _oracle_dg(inp, "fp32")
    K, N = inp["w_g"].shape
    init = torch.linspace(-1.0, 1.0, K * N).reshape(K, N)
    _w_case(inp["x"], dg, dfc, "fp32", dw0=init)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_x_stage_empty_contraction_writes_zero(dt):
    dev = device()
    M, K = 33, 16
    tdt = DTYPES[dt]
    dx = torch.full((M, K), 3.0, dtype=tdt, device=dev)
    e = torch.empty(M, 0, dtype=tdt, device=dev)
    w = torch.empty(K, 0, dtype=tdt, device=dev)
    note(f"x stage N=0 {dt}")
    swg.swiglu_bwd_x(e, e, w, w, dx)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dx).item() == 0


def test_chained_b_w_x_on_ragged_batch():
    """GPU b feeds GPU w and x; compared with the oracle chained in float64."""
    dev = device()
    inp = swiglu_inputs("ragged", dtype="bf16")
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    d = {k: v.to(dev) for k, v in inp.items()}
    dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
    db_g = torch.zeros(N, dtype=torch.bfloat16, device=dev)
    db_fc = torch.zeros_like(db_g)
    dw_g = torch.zeros(K, N, dtype=torch.bfloat16, device=dev)
    dw_fc = torch.zeros_like(dw_g)
    dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
    note("chained b -> w -> x ragged")
    swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc)
    swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc)
    swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx)
    torch.cuda.synchronize()
    dy64, g64, fc64, x64 = (to64(inp[k]) for k in ("dy", "g", "fc", "x"))
    wg64, wf64 = to64(inp["w_g"]), to64(inp["w_fc"])
    ref = R.swiglu_bwd_ref(dy64, x64, wg64, wf64, g64, fc64)
    # rounding models: dg, dfc element-wise; db from the fp32 values of dg / dfc; dw and dx
    # from the bf16 dg / dfc the b stage stored (one storage rounding per operand element)
    adg, adfc = np.abs(ref["dg"]), np.abs(ref["dfc"])
    ax = np.abs(x64)
    models = {"dg": dg_abs_model(dy64, g64, fc64), "dfc": dfc_abs_model(dy64, g64),
              "db_g": sum_abs_model(adg.sum(0)), "db_fc": sum_abs_model(adfc.sum(0)),
              "dw_g": chained_abs_model(ax.T @ adg, "bf16"),
              "dw_fc": chained_abs_model(ax.T @ adfc, "bf16"),
              "dx": chained_abs_model(adg @ np.abs(wg64).T + adfc @ np.abs(wf64).T, "bf16")}
    got = {"dg": dg, "dfc": dfc, "db_g": db_g, "db_fc": db_fc, "dw_g": dw_g, "dw_fc": dw_fc,
           "dx": dx}
    for k, v in got.items():
        compare(f"chained {k}", v.cpu(), ref[k], "bf16", model_abs=models[k])


# Gate values from the saturated tails to zero, within each dtype's finite range: sigma
# and 1 - sigma underflow (g -> -inf: dg -> 0, dfc -> 0) or reach 1 and 0 (g -> +inf:
# dg -> dy fc, dfc -> dy g), and g = +-0 gives dg = dy fc / 2, dfc = 0.
_EXTREME_G = {
    "bf16": [-3.0e38, -1.0e4, -700.0, -100.0, -88.5, -30.0, -17.0, -1e-30, -0.0,
             0.0, 1e-30, 17.0, 30.0, 88.5, 100.0, 700.0, 1.0e4, 3.0e38],
    "fp16": [-6.0e4, -1.0e4, -700.0, -100.0, -88.5, -30.0, -17.0, -1e-7, -0.0,
             0.0, 1e-7, 17.0, 30.0, 88.5, 100.0, 700.0, 1.0e4, 6.0e4],
    "fp32": [-3.0e38, -1.0e4, -700.0, -100.0, -88.5, -30.0, -17.0, -1e-40, -0.0,
             0.0, 1e-40, 17.0, 30.0, 88.5, 100.0, 700.0, 1.0e4, 3.0e38],
}


def _extreme_b_inputs(dt, M=257, N=144, seed=61):
    """dy ~ N(0,1) 1e-3 and fc ~ N(0,1); every row of g a seeded arrangement of the
    extreme gate values (so dfc = dy g sigma(g) stays finite: |dy g| < 1e36)."""
    gen = torch.Generator().manual_seed(seed)
    vals = torch.tensor(_EXTREME_G[dt], dtype=torch.float64)
    idx = torch.randint(0, len(vals), (M, N), generator=gen)
    tdt = DTYPES[dt]
    return {"dy": (torch.randn(M, N, generator=gen) * 1e-3).to(tdt),
            "g": vals[idx].to(tdt),
            "fc": torch.randn(M, N, generator=gen).to(tdt)}


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_b_stage_saturated_gate_values(dt):
    """Extreme but finite g: outputs finite and within the tolerances of the oracle."""
    _b_case(_extreme_b_inputs(dt), dt)


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_b_stage_non_finite_gate_values(dt):
    """g = +-inf or NaN in a few positions: dg and dfc are NaN or +-inf exactly where the
    oracle's float64 values are (SiLU'(+-inf) takes inf * 0 = NaN, as torch's
    silu_backward does; dfc = dy * (+inf) * 1 = +-inf, dy * (-inf) * 0 = NaN), and every
    other element and every column sum of finite columns matches the oracle."""
    dev = device()
    inp = _extreme_b_inputs(dt, M=129, N=64, seed=62)
    g = inp["g"].clone()
    bad = [(0, 0, float("inf")), (5, 9, float("-inf")), (64, 17, float("nan")),
           (128, 63, float("nan"))]
    for r, c, v in bad:
        g[r, c] = v
    inp["g"] = g
    M, N = g.shape
    tdt = DTYPES[dt]
    dy, gg, fc = (inp[k].to(dev) for k in ("dy", "g", "fc"))
    dg, dfc = torch.empty_like(dy), torch.empty_like(dy)
    db_g, db_fc = torch.zeros(N, dtype=tdt, device=dev), torch.zeros(N, dtype=tdt, device=dev)
    note(f"b stage non-finite g {dt}")
    swg.swiglu_bwd_b(dy, gg, fc, dg, dfc, db_g, db_fc)
    torch.cuda.synchronize()
    dy64, g64, fc64 = to64(inp["dy"]), to64(g), to64(inp["fc"])
    with np.errstate(all="ignore"):
        rdg, rdfc, rbg, rbf = R.b_ref(dy64, g64, fc64)
        models = {"dg": dg_abs_model(dy64, g64, fc64), "dfc": dfc_abs_model(dy64, g64)}
    for name, got, ref in (("dg", dg, rdg), ("dfc", dfc, rdfc), ("db_g", db_g, rbg),
                           ("db_fc", db_fc, rbf)):
        got = to64(got.cpu())
        fin = np.isfinite(ref)
        assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{name}: NaN positions"
        assert np.array_equal(np.isposinf(got), np.isposinf(ref)), f"{name}: +inf positions"
        assert np.array_equal(np.isneginf(got), np.isneginf(ref)), f"{name}: -inf positions"
        assert (~fin).any() or name.startswith("db"), f"{name}: no non-finite case exercised"
        if name in models:
            compare(name, got[fin], ref[fin], dt, model_abs=models[name][fin])
        else:
            terms = rdg if name == "db_g" else rdfc
            absum = np.abs(np.where(np.isfinite(terms), terms, 0.0)).sum(0)
            compare(name, got[fin], ref[fin], dt, model_abs=sum_abs_model(absum[fin]))


def test_bitwise_deterministic_reruns():
    dev = device()
    inp = swiglu_inputs("ragged", dtype="bf16")
    d = {k: v.to(dev) for k, v in inp.items()}
    M, N = inp["dy"].shape
    K = inp["x"].shape[1]
    outs = []
    for _ in range(2):
        dg, dfc = torch.empty_like(d["dy"]), torch.empty_like(d["dy"])
        db_g = torch.zeros(N, dtype=torch.bfloat16, device=dev)
        db_fc = torch.zeros_like(db_g)
        dw_g = torch.zeros(K, N, dtype=torch.bfloat16, device=dev)
        dw_fc = torch.zeros_like(dw_g)
        dx = torch.empty(M, K, dtype=torch.bfloat16, device=dev)
        swg.swiglu_bwd_b(d["dy"], d["g"], d["fc"], dg, dfc, db_g, db_fc)
        swg.swiglu_bwd_w(d["x"], dg, dfc, dw_g, dw_fc)
        swg.swiglu_bwd_x(dg, dfc, d["w_g"], d["w_fc"], dx)
        torch.cuda.synchronize()
        outs.append([t.view(torch.int16).cpu() for t in (dg, dfc, db_g, db_fc, dw_g, dw_fc, dx)])
    for a, b in zip(*outs):
        assert torch.equal(a, b)
