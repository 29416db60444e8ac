"""The C ABI from a plain C program: tests/c_abi_program.c allocates device memory with the
HIP runtime's C API, runs b -> w -> x and the Swish gradient through libswiglu_bwd.so (no
Python or torch in that process) and writes its outputs to files, which are compared here
with the float64 oracle (the tiny workload, chained, and a ragged-length Swish input)."""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle.ref as R
import swish_activation_backward_amd as swg
from gpu_util import device, note
from parity import (chained_abs_model, compare, dfc_abs_model, dg_abs_model, sum_abs_model,
                    swish_abs_model, to64)
from workloads.gen import swiglu_inputs, swish_inputs

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _write(t, path):
    t.contiguous().view(torch.int16).numpy().tofile(path)


def _read(path, shape):
    raw = np.fromfile(path, dtype=np.int16)
    return torch.from_numpy(raw).view(torch.bfloat16).reshape(shape)


def test_c_program_runs_the_path_through_the_c_abi(tmp_path):
    device()
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not installed")
    libdir = os.path.dirname(swg.library_path())
    exe = tmp_path / "c_abi_program"
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c_abi_program.c"), "-o", str(exe),
           "-L", libdir, "-lswiglu_bwd", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{libdir}", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]

    inp = swiglu_inputs("tiny", dtype="bf16")
    M, K = inp["x"].shape
    N = inp["dy"].shape[1]
    L = 100003
    sw = swish_inputs("bf16", L=L, seed=71)
    for name in ("x", "dy", "g", "fc", "w_g", "w_fc"):
        _write(inp[name], tmp_path / f"{name}.bin")
    _write(sw["grad"], tmp_path / "grad.bin")
    _write(sw["x"], tmp_path / "sx.bin")
    note(f"C program: b -> w -> x M={M} K={K} N={N} and swish_grad L={L} (child process)")
    run = subprocess.run([str(exe), str(tmp_path), str(M), str(K), str(N), str(L)],
                         capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr[-3000:]
    assert "c_abi_program ok" in run.stdout

    shapes = {"dg": (M, N), "dfc": (M, N), "db_g": (N,), "db_fc": (N,), "dw_g": (K, N),
              "dw_fc": (K, N), "dx": (M, K)}
    got = {k: _read(tmp_path / f"{k}.bin", s) for k, s in shapes.items()}
    dy64, g64, fc64, x64 = (to64(inp[k]) for k in ("dy", "g", "fc", "x"))
    wg64, wf64 = to64(inp["w_g"]), to64(inp["w_fc"])
    ref = R.swiglu_bwd_ref(dy64, x64, wg64, wf64, g64, fc64)
    adg, adfc = np.abs(ref["dg"]), np.abs(ref["dfc"])
    ax = np.abs(x64)
    models = {"dg": dg_abs_model(dy64, g64, fc64), "dfc": dfc_abs_model(dy64, g64),
              "db_g": sum_abs_model(adg.sum(0)), "db_fc": sum_abs_model(adfc.sum(0)),
              "dw_g": chained_abs_model(ax.T @ adg, "bf16"),
              "dw_fc": chained_abs_model(ax.T @ adfc, "bf16"),
              "dx": chained_abs_model(adg @ np.abs(wg64).T + adfc @ np.abs(wf64).T, "bf16")}
    for k, v in got.items():
        compare(f"C program {k}", v, ref[k], "bf16", model_abs=models[k])

    gx = _read(tmp_path / "gx.bin", (L,))
    g64s, x64s = to64(sw["grad"]), to64(sw["x"])
    compare("C program swish_grad", gx, R.swish_grad_ref(g64s, x64s, 1.702), "bf16",
            model_abs=swish_abs_model(g64s, x64s, 1.702))
