"""GPU parity past 2^31 elements per tensor: the b stage, the w and x stages, the fused
w + x pass, the forward and swish_grad on tensors whose element offsets do not fit 32 bits (and, for
swish_grad, long enough that its grid strides: more than 2^20 workgroups of vectors).

Inputs are a seeded block of P rows (P odd, so no 2^k-element wrap of an offset lands on
an equal value) drawn with the workload recipe and repeated down the rows on the device.
Every output is then checked without running the oracle on billions of elements:
  * the outputs of the first P rows against the oracle, element by element;
  * every later row bit-identical to its counterpart in the first block (each output
    row of these stages depends only on the same input row, through the same
    arithmetic in the same order);
  * the sums over M (db, dW) against the oracle's exact value for the repeated block:
    q times the block's sum plus the partial block's.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import device, note, oracle_b_chunked, oracle_w_chunked, oracle_x_rows
from parity import compare, forward_abs_models, sum_abs_model, swish_abs_model, to64
from workloads.gen import DTYPES, SwiGLUShape, swiglu_inputs, swish_inputs

pytestmark = pytest.mark.gpu

TWO31 = 1 << 31
# (P, M, N) of the b-stage case, (P, M, K, N) of the GEMM case, P of the swish_grad cases
B_CASE = (4099, (1 << 21) + 77, 1048)
GEMM_CASE = (4099, (1 << 20) + 77, 2048, 512)
FWD_CASE = (4099, (1 << 20) + 77, 2048, 2048)
SWISH_P = 1000003
SWISH_CASES = [("bf16", TWO31 + (1 << 21) + 37), ("fp32", (1 << 30) + (1 << 20) + 5)]


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info(device())
    if free < nbytes:
        pytest.skip(f"needs {nbytes / 2**30:.0f} GiB of free device memory")


def _tile_rows(block, rows, dev):
    """`block` repeated down its first dimension to `rows` rows, on the device."""
    reps = -(-rows // block.shape[0])
    dims = (reps,) + (1,) * (block.dim() - 1)
    return block.to(dev).repeat(*dims)[:rows]


def _assert_periodic(name, t, P, chunk=64):
    """Every P-row block of t is bit-identical to the first (the last may be partial)."""
    iv = t.view({2: torch.int16, 4: torch.int32}[t.element_size()])
    head = iv[:P]
    M = iv.shape[0]
    q = M // P
    for k0 in range(1, q, chunk):
        k1 = min(q, k0 + chunk)
        body = iv[k0 * P:k1 * P].reshape((k1 - k0, P) + tuple(iv.shape[1:]))
        assert torch.equal(body, head.unsqueeze(0).expand_as(body)), f"{name}: blocks {k0}..{k1}"
    if M > q * P:
        assert torch.equal(iv[q * P:], head[:M - q * P]), f"{name}: partial block"


def _block_sum(full, part, q):
    """q repetitions of a block's sum plus the sum over the partial block's rows."""
    return q * full + part


def test_b_stage_past_2_31_elements():
    """M = 2^21 + 77 rows of N = 1048 (2.2e9 elements per tensor, bf16)."""
    dev = device()
    (P, M, N), dt = B_CASE, "bf16"
    assert M * N > TWO31
    _need(5 * M * N * 2 + (1 << 30))
    blk = swiglu_inputs(SwiGLUShape("large_b", 41, P, 64, N), dtype=dt)
    tdt = DTYPES[dt]
    dy, g, fc = (_tile_rows(blk[k], M, dev) for k in ("dy", "g", "fc"))
    dg, dfc = torch.empty_like(dy), torch.empty_like(dy)
    db_g = torch.zeros(N, dtype=tdt, device=dev)
    db_fc = torch.zeros_like(db_g)
    note(f"b stage M={M} N={N} {dt} (2^31+ elements)")
    swg.swiglu_bwd_b(dy, g, fc, dg, dfc, db_g, db_fc)
    torch.cuda.synchronize()
    del dy, g, fc
    q, rem = divmod(M, P)
    full = oracle_b_chunked(blk["dy"], blk["g"], blk["fc"], gpu=(dg[:P].cpu(), dfc[:P].cpu()))
    full["check_dg"].result()
    full["check_dfc"].result()
    part = oracle_b_chunked(blk["dy"][:rem], blk["g"][:rem], blk["fc"][:rem])
    for name, t in (("dg", dg), ("dfc", dfc)):
        _assert_periodic(name, t, P)
    for key, ab, got in (("db_g", "abs_g", db_g), ("db_fc", "abs_fc", db_fc)):
        ref = _block_sum(full[key], part[key], q)
        compare(key, got.cpu(), ref, dt, model_abs=sum_abs_model(_block_sum(full[ab], part[ab], q)))
    del dg, dfc
    torch.cuda.empty_cache()


def test_gemm_stages_past_2_31_elements():
    """x and dx of M = 2^20 + 77 rows by K = 2048 (2.1e9 elements), N = 512, bf16: the
    x stage, the w stage and the fused pass (whose dx must equal the x stage's bits)."""
    dev = device()
    (P, M, K, N), dt = GEMM_CASE, "bf16"
    assert M * K > TWO31
    _need(3 * M * K * 2 + 2 * M * N * 2 + (2 << 30))
    tdt = DTYPES[dt]
    blk = swiglu_inputs(SwiGLUShape("large_gemm", 43, P, K, N), dtype=dt)
    ob = oracle_b_chunked(blk["dy"], blk["g"], blk["fc"], store_dtype=tdt)
    bdg, bdfc = ob["dg"], ob["dfc"]              # the oracle's rounded dg / dfc block
    x = _tile_rows(blk["x"], M, dev)
    dg, dfc = _tile_rows(bdg, M, dev), _tile_rows(bdfc, M, dev)
    w_g, w_fc = blk["w_g"].to(dev), blk["w_fc"].to(dev)
    q, rem = divmod(M, P)

    dx = torch.empty(M, K, dtype=tdt, device=dev)
    note(f"x stage M={M} K={K} N={N} {dt} (2^31+ elements)")
    swg.swiglu_bwd_x(dg, dfc, w_g, w_fc, dx)
    torch.cuda.synchronize()
    ref, a = oracle_x_rows(bdg, bdfc, blk["w_g"], blk["w_fc"], slice(None))
    compare("dx[:P]", dx[:P].cpu(), ref, dt, model_abs=sum_abs_model(a))
    _assert_periodic("dx", dx, P)

    rg, rf, ag, af = oracle_w_chunked(blk["x"], bdg, bdfc)
    pg, pf, pag, paf = oracle_w_chunked(blk["x"][:rem], bdg[:rem], bdfc[:rem])
    want = {"dw_g": (_block_sum(rg, pg, q), _block_sum(ag, pag, q)),
            "dw_fc": (_block_sum(rf, pf, q), _block_sum(af, paf, q))}

    dw_g = torch.zeros(K, N, dtype=tdt, device=dev)
    dw_fc = torch.zeros_like(dw_g)
    note(f"w stage M={M} K={K} N={N} {dt} (2^31+ elements)")
    swg.swiglu_bwd_w(x, dg, dfc, dw_g, dw_fc)
    torch.cuda.synchronize()
    for name, got in (("dw_g", dw_g), ("dw_fc", dw_fc)):
        compare(name, got.cpu(), want[name][0], dt, model_abs=sum_abs_model(want[name][1]))

    dx2 = torch.empty_like(dx)
    dw_g.zero_()
    dw_fc.zero_()
    note(f"fused w+x M={M} K={K} N={N} {dt} (2^31+ elements)")
    swg.swiglu_bwd_wx(x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx2)
    torch.cuda.synchronize()
    assert torch.equal(dx2.view(torch.int16), dx.view(torch.int16)), "fused dx"
    for name, got in (("dw_g", dw_g), ("dw_fc", dw_fc)):
        compare(f"fused {name}", got.cpu(), want[name][0], dt,
                model_abs=sum_abs_model(want[name][1]))
    del x, dg, dfc, dx, dx2
    torch.cuda.empty_cache()


def test_forward_past_2_31_elements():
    """x, g, fc and y of M = 2^20 + 77 rows by 2048 columns (2.1e9 elements each), bf16."""
    dev = device()
    (P, M, K, N), dt = FWD_CASE, "bf16"
    assert M * K > TWO31 and M * N > TWO31
    _need(M * K * 2 + 3 * M * N * 2 + (1 << 30))
    tdt = DTYPES[dt]
    blk = swiglu_inputs(SwiGLUShape("large_fwd", 53, P, K, N), dtype=dt, with_forward=False)
    x = _tile_rows(blk["x"], M, dev)
    g, fc, y = (torch.empty(M, N, dtype=tdt, device=dev) for _ in range(3))
    note(f"forward M={M} K={K} N={N} {dt} (2^31+ elements)")
    swg.swiglu_fwd(x, blk["w_g"].to(dev), blk["w_fc"].to(dev), blk["b_g"].to(dev),
                   blk["b_fc"].to(dev), g, fc, y)
    torch.cuda.synchronize()
    del x
    xr = to64(blk["x"])
    rg, rf, ry = R.swiglu_forward_ref(xr, to64(blk["w_g"]), to64(blk["b_g"]), to64(blk["w_fc"]),
                                      to64(blk["b_fc"]))
    eg, ef, ey = forward_abs_models(xr, blk["w_g"], blk["w_fc"], blk["b_g"], blk["b_fc"], rg, rf)
    for name, t, ref, model in (("g", g, rg, eg), ("fc", fc, rf, ef), ("y", y, ry, ey)):
        compare(f"{name}[:P]", t[:P].cpu(), ref, dt, model_abs=model)
        _assert_periodic(name, t, P)
    del g, fc, y
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dt,n", SWISH_CASES)
def test_swish_grad_past_2_20_workgroups(dt, n):
    """bf16 past 2^31 elements and fp32 past 2^30 (4 GiB per tensor): both have more than
    2^20 workgroups' worth of 16-byte vectors, so the grid strides; ragged tails."""
    dev = device()
    P, beta = SWISH_P, 1.702
    esize = torch.empty((), dtype=DTYPES[dt]).element_size()
    _need(3 * n * esize + (1 << 30))
    blk = swish_inputs(dt, L=P, seed=47)
    grad, x = _tile_rows(blk["grad"], n, dev), _tile_rows(blk["x"], n, dev)
    note(f"swish_grad n={n} {dt} beta={beta} (grid-stride path)")
    out = swg.swish_grad(grad, x, beta=beta)
    torch.cuda.synchronize()
    del grad, x
    g64, x64 = blk["grad"].double().numpy(), blk["x"].double().numpy()
    ref, model = R.swish_grad_ref(g64, x64, beta), swish_abs_model(g64, x64, beta)
    compare("swish_grad[:P]", out[:P].cpu(), ref, dt, model_abs=model)
    # the vector body is periodic bit for bit; the n % 16-byte scalar tail is compared
    # with the oracle value of its position in the block
    nv = n - n % (16 // esize)
    _assert_periodic("swish_grad", out[:nv], P, chunk=256)
    pos = np.arange(nv, n) % P
    compare("swish_grad tail", out[nv:].cpu(), ref[pos], dt, model_abs=model[pos])
    del out
    torch.cuda.empty_cache()
