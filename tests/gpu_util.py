"""Helpers for the GPU parity tests: device handling, guard-band canaries, and the
chunked drive of the float64 oracle over large workloads."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle.ref as R
from parity import Checker, dfc_abs_model, dg_abs_model, sum_abs_model, to64

# numpy releases the GIL inside its loops: row blocks of the oracle run on a thread pool
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))

SENTINEL_BITS = {torch.bfloat16: 0x7FA5, torch.float16: 0x7DA5, torch.float32: 0x7FA5A5A5}


def device():
    if not torch.cuda.is_available():
        pytest.fail("a GPU test ran without a visible GPU")
    return torch.device("cuda", 0)


def note(msg):
    """Progress line naming the case, flushed before the GPU step it announces."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


class Guarded:
    """A device buffer with `pad` sentinel elements on both sides of the payload."""

    def __init__(self, shape, dtype, dev, pad=64, fill=None):
        n = int(np.prod(shape)) if len(shape) else 1
        itype = {2: torch.int16, 4: torch.int32}[torch.empty((), dtype=dtype).element_size()]
        self.raw = torch.empty(n + 2 * pad, dtype=dtype, device=dev)
        self.raw.view(itype).fill_(SENTINEL_BITS[dtype])   # a NaN pattern in each dtype
        self.pad, self.n, self.shape, self.itype = pad, n, tuple(shape), itype
        self.t = self.raw[pad:pad + n].view(*shape)
        if fill is not None:
            self.t.copy_(fill)

    def check(self):
        raw = self.raw.view(self.itype).cpu()
        want = raw[0].item()
        head, tail = raw[:self.pad], raw[self.pad + self.n:]
        assert torch.all(head == want) and torch.all(tail == want), "guard band overwritten"


def rne(a64, dtype):
    """Round a float64 array to the storage dtype (nearest even) as a CPU tensor."""
    return torch.from_numpy(np.ascontiguousarray(a64)).to(dtype)


def oracle_b_chunked(dy, g, fc, db_g0=None, db_fc0=None, rows=4096, gpu=None, dtype="bf16",
                     store_dtype=None):
    """Run the oracle's b stage over row blocks (on a thread pool).

    Returns a dict with db_g, db_fc (float64, initial values added), abs_g / abs_fc (the
    column sums of |dg| / |dfc|) and, when `store_dtype` is given, the oracle's dg / dfc
    rounded to it (CPU tensors).  If `gpu` = (dg_gpu, dfc_gpu) CPU tensors is given they
    are compared block by block and the two Checkers are returned as check_dg/check_dfc.
    """
    M, N = dy.shape
    out_g = torch.empty((M, N), dtype=store_dtype) if store_dtype is not None else None
    out_fc = torch.empty((M, N), dtype=store_dtype) if store_dtype is not None else None

    def block(r0):
        r1 = min(M, r0 + rows)
        cdy, cg, cfc = to64(dy[r0:r1]), to64(g[r0:r1]), to64(fc[r0:r1])
        dgv, dfcv, sg, sf = R.b_ref(cdy, cg, cfc)
        part = {"sg": sg, "sf": sf, "ag": np.abs(dgv).sum(0), "af": np.abs(dfcv).sum(0)}
        if out_g is not None:
            out_g[r0:r1] = rne(dgv, store_dtype)
            out_fc[r0:r1] = rne(dfcv, store_dtype)
        if gpu is not None:
            part["cg"] = Checker("dg", dtype).add(gpu[0][r0:r1], dgv, dg_abs_model(cdy, cg, cfc))
            part["cf"] = Checker("dfc", dtype).add(gpu[1][r0:r1], dfcv, dfc_abs_model(cdy, cg))
        return part

    with ThreadPoolExecutor(WORKERS) as ex:
        parts = list(ex.map(block, range(0, M, rows)))
    db_g = np.zeros(N) if db_g0 is None else to64(db_g0).copy()
    db_fc = np.zeros(N) if db_fc0 is None else to64(db_fc0).copy()
    abs_g, abs_fc = np.zeros(N), np.zeros(N)
    ck_g = Checker("dg", dtype) if gpu is not None else None
    ck_fc = Checker("dfc", dtype) if gpu is not None else None
    for p in parts:                 # fixed (row-block) order
        db_g += p["sg"]
        db_fc += p["sf"]
        abs_g += p["ag"]
        abs_fc += p["af"]
        if gpu is not None:
            ck_g.merge(p["cg"])
            ck_fc.merge(p["cf"])
    res = {"db_g": db_g, "db_fc": db_fc, "abs_g": abs_g, "abs_fc": abs_fc,
           "dg": out_g, "dfc": out_fc}
    if gpu is not None:
        res["check_dg"], res["check_dfc"] = ck_g, ck_fc
    return res


def oracle_w_chunked(x, dg, dfc, cols=None, rows=16384):
    """dw = x^T [dg | dfc] (restricted to `cols` of N if given) and the magnitude sums
    |x|^T |dg|, summed over row blocks of the plain oracle."""
    M, K = x.shape
    N = dg.shape[1]
    sel = slice(None) if cols is None else cols
    width = N if cols is None else len(cols)
    dw_g, dw_fc = np.zeros((K, width)), np.zeros((K, width))
    a_g, a_fc = np.zeros((K, width)), np.zeros((K, width))
    for r0 in range(0, M, rows):
        r1 = min(M, r0 + rows)
        cx = to64(x[r0:r1])
        cg, cf = to64(dg[r0:r1])[:, sel], to64(dfc[r0:r1])[:, sel]
        pg, pf = R.w_ref(cx, cg, cf)
        dw_g += pg
        dw_fc += pf
        ax = np.abs(cx)
        a_g += ax.T @ np.abs(cg)
        a_fc += ax.T @ np.abs(cf)
    return dw_g, dw_fc, a_g, a_fc


def oracle_x_rows(dg, dfc, w_g, w_fc, rows_idx):
    """dx on the selected rows, with the magnitude sum |dg||W_g|^T + |dfc||W_fc|^T."""
    cg, cf = to64(dg[rows_idx]), to64(dfc[rows_idx])
    wg, wf = to64(w_g), to64(w_fc)
    dx = R.x_ref(cg, cf, wg, wf)
    a = np.abs(cg) @ np.abs(wg).T + np.abs(cf) @ np.abs(wf).T
    return dx, a


__all__ = ["device", "note", "Guarded", "rne", "oracle_b_chunked", "oracle_w_chunked",
           "oracle_x_rows", "sum_abs_model"]
