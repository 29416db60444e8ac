"""Seeded synthetic inputs for the SwiGLU backward and Swish-gradient workloads.

This module only draws random numbers and rounds them to the storage dtype; it holds
none of the backward method's arithmetic.  Both the GPU path's tests/bench and the CPU
oracle receive the exact tensors built here.

Shapes and distributions follow the workloads the pages describe:
  * the Fused SwiGLU backward page (PyPTO-Gym, hnwysp.cn), section "test cases":
    M=220000, K=512, N=1024, bf16, inputs scaled by 1/sqrt(m) and weights by
    1/sqrt(k), seed 0;
  * the SwishGrad/aclnnSwishBackward page (ops-nn, bhfrc.com), section 1.3 and 2.4:
    fp32/fp16/bf16 tensors with a scalar fp32 beta.

Recipe (the pages fix neither the RNG nor the draw order; this is the reading taken):
  * one torch CPU ``Generator`` seeded with the workload seed;
  * fp32 draws in the order x, dy, w_g, w_fc, b_g, b_fc (SwiGLU) or grad, x (Swish);
  * "N(0, s)" reads s as the standard deviation;
  * every tensor is rounded to the storage dtype with round-to-nearest-even;
  * g and fc come from the forward pass, computed in fp32 from the *rounded*
    bf16 x, w and b, then rounded to bf16.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch

__all__ = [
    "SwiGLUShape", "SWIGLU_WORKLOADS", "SWISH_WORKLOAD", "SWISH_CONTEXT", "swiglu_inputs",
    "swish_inputs", "sha256_of", "DTYPES",
]

DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


@dataclass(frozen=True)
class SwiGLUShape:
    name: str
    seed: int
    M: int
    K: int
    N: int


# The SwiGLU workloads: tiny, ragged batch (M = 2^13 - 1), the pages' large-batch FFN
# test shape, and an LLM-sized FFN.
SWIGLU_WORKLOADS = {
    "tiny": SwiGLUShape("tiny", 0, 256, 64, 128),
    "ragged": SwiGLUShape("ragged", 2, 8191, 512, 1024),
    "ffn_220k": SwiGLUShape("ffn_220k", 0, 220000, 512, 1024),
    "llm_ffn": SwiGLUShape("llm_ffn", 3, 16384, 4096, 14336),
}

# The stand-alone Swish-gradient workload: length 2^24 + 37 (ragged tail),
# three storage dtypes and three beta values.
SWISH_WORKLOAD = {"seed": 1, "L": (1 << 24) + 37, "betas": (1.0, 1.702, 0.5),
                  "dtypes": ("fp32", "fp16", "bf16")}


# The one timed Swish-gradient case on the pages (the Ascend C custom-operator page,
# performance table): an fp16 activation of shape [32, 64, 56, 56] (6,422,528 elements),
# plain SiLU backward (beta = 1).  Drawn with the Swish workload's distributions.
SWISH_CONTEXT = {"seed": 4, "shape": (32, 64, 56, 56), "dtype": "fp16", "beta": 1.0}


def _randn(gen: torch.Generator, shape, scale: float) -> torch.Tensor:
    t = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t


def swiglu_inputs(shape: SwiGLUShape | str, dtype: str = "bf16",
                  with_forward: bool = True, M: int | None = None) -> dict:
    """Draw x, dy, w_g, w_fc, b_g, b_fc and (optionally) g, fc for one workload.

    Returns CPU tensors in the storage dtype.  ``M`` overrides the batch size
    (the draws then use the overridden M for the 1/sqrt(M) scaling).
    """
    if isinstance(shape, str):
        shape = SWIGLU_WORKLOADS[shape]
    M = shape.M if M is None else M
    K, N = shape.K, shape.N
    tdt = DTYPES[dtype]
    gen = torch.Generator().manual_seed(shape.seed)
    inv_sqrt_m = 1.0 / math.sqrt(max(M, 1))
    inv_sqrt_k = 1.0 / math.sqrt(K)
    out = {}
    out["x"] = _randn(gen, (M, K), inv_sqrt_m).to(tdt)
    out["dy"] = _randn(gen, (M, N), inv_sqrt_m).to(tdt)
    out["w_g"] = _randn(gen, (K, N), inv_sqrt_k).to(tdt)
    out["w_fc"] = _randn(gen, (K, N), inv_sqrt_k).to(tdt)
    out["b_g"] = _randn(gen, (N,), 0.02).to(tdt)
    out["b_fc"] = _randn(gen, (N,), 0.02).to(tdt)
    if with_forward:
        # Forward pass (input generation only): fp32 from the rounded tensors.
        xf = out["x"].float()
        out["g"] = torch.addmm(out["b_g"].float(), xf, out["w_g"].float()).to(tdt)
        out["fc"] = torch.addmm(out["b_fc"].float(), xf, out["w_fc"].float()).to(tdt)
    return out


def swish_inputs(dtype: str, L: int | None = None, seed: int | None = None) -> dict:
    """grad ~ N(0,1), x ~ N(0,3) drawn in fp32 (grad first), rounded to ``dtype``."""
    seed = SWISH_WORKLOAD["seed"] if seed is None else seed
    L = SWISH_WORKLOAD["L"] if L is None else L
    gen = torch.Generator().manual_seed(seed)
    grad = _randn(gen, (L,), 1.0)
    x = _randn(gen, (L,), 3.0)
    tdt = DTYPES[dtype]
    return {"grad": grad.to(tdt), "x": x.to(tdt)}


def sha256_of(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's raw bytes (row-major, storage dtype)."""
    t = t.detach().contiguous().cpu()
    raw = t.view(torch.uint8) if t.element_size() > 0 and t.numel() > 0 else t
    return hashlib.sha256(raw.numpy().tobytes()).hexdigest()
