"""Drop-in training use: a ``torch.autograd.Function`` and an ``nn.Module`` for the SwiGLU
feed-forward gate whose forward and backward both run in the library's kernels.

    y = SiLU(x W_g + b_g) * (x W_fc + b_fc)

Forward: ``swiglu_fwd`` (g, fc and y from one fused GEMM); g and fc are saved for the
backward, which runs the three stages of the Fused SwiGLU backward page's call chain
(b -> w -> x): ``swiglu_bwd_b`` (dg, dfc, db), then, when both dW and dx are needed, the
fused ``swiglu_bwd_wx`` (both GEMMs over [dg | dfc] from one launch in bf16 / fp16),
otherwise ``swiglu_bwd_w`` (dW) or ``swiglu_bwd_x`` (dx).  The pattern is a custom operator whose backward hook calls a hand-written gradient
kernel (the Ascend C custom-backward page, "突破自动微分瓶颈: 基于 Ascend C 的高性能自定义反向传播
算子实战", section 4.2, Python-side registration); the weight layout [K, N] is the SwiGLU
page's.  Leading dimensions of x are flattened into M.
"""
from __future__ import annotations

import math

import torch

from . import _lib


class SwiGLUFunction(torch.autograd.Function):
    """x [M, K], w_g / w_fc [K, N], b_g / b_fc [N] or None -> y [M, N] (bf16, fp16 or fp32,
    contiguous, on the GPU)."""

    @staticmethod
    def forward(ctx, x, w_g, w_fc, b_g, b_fc):
        M, N = x.shape[0], w_g.shape[1]
        g = torch.empty(M, N, dtype=x.dtype, device=x.device)
        fc = torch.empty_like(g)
        y = torch.empty_like(g)
        _lib.swiglu_fwd(x, w_g, w_fc, b_g, b_fc, g, fc, y)
        ctx.save_for_backward(x, w_g, w_fc, g, fc)
        ctx.has_bias = (b_g is not None, b_fc is not None)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, w_g, w_fc, g, fc = ctx.saved_tensors
        dy = dy.contiguous()
        M, N = g.shape
        K = x.shape[1]
        dg, dfc = torch.empty_like(g), torch.empty_like(fc)
        db_g = torch.zeros(N, dtype=g.dtype, device=g.device)
        db_fc = torch.zeros_like(db_g)
        _lib.swiglu_bwd_b(dy, g, fc, dg, dfc, db_g, db_fc)
        dx = dw_g = dw_fc = None
        need_w = ctx.needs_input_grad[1] or ctx.needs_input_grad[2]
        if need_w and ctx.needs_input_grad[0]:
            dw_g = torch.zeros(K, N, dtype=g.dtype, device=g.device)
            dw_fc = torch.zeros_like(dw_g)
            dx = torch.empty(M, K, dtype=x.dtype, device=x.device)
            _lib.swiglu_bwd_wx(x, dg, dfc, w_g, w_fc, dw_g, dw_fc, dx)
            return (dx, dw_g, dw_fc, db_g if ctx.has_bias[0] else None,
                    db_fc if ctx.has_bias[1] else None)
        if need_w:
            dw_g = torch.zeros(K, N, dtype=g.dtype, device=g.device)
            dw_fc = torch.zeros_like(dw_g)
            _lib.swiglu_bwd_w(x, dg, dfc, dw_g, dw_fc)
        if ctx.needs_input_grad[0]:
            dx = torch.empty(M, K, dtype=x.dtype, device=x.device)
            _lib.swiglu_bwd_x(dg, dfc, w_g, w_fc, dx)
        return (dx, dw_g, dw_fc, db_g if ctx.has_bias[0] else None,
                db_fc if ctx.has_bias[1] else None)


def swiglu(x, w_g, w_fc, b_g=None, b_fc=None):
    """SwiGLU gate over the last dimension of x (any leading shape)."""
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1]).contiguous()
    y = SwiGLUFunction.apply(x2, w_g, w_fc, b_g, b_fc)
    return y.view(*lead, w_g.shape[1])


class SwiGLU(torch.nn.Module):
    """Parameters w_g, w_fc [in_features, hidden] and optional biases [hidden]; forward(x)
    maps [..., in_features] to [..., hidden]."""

    def __init__(self, in_features, hidden, bias=True, device=None, dtype=torch.bfloat16):
        super().__init__()
        kw = {"device": device, "dtype": dtype}
        self.w_g = torch.nn.Parameter(torch.empty(in_features, hidden, **kw))
        self.w_fc = torch.nn.Parameter(torch.empty(in_features, hidden, **kw))
        if bias:
            self.b_g = torch.nn.Parameter(torch.zeros(hidden, **kw))
            self.b_fc = torch.nn.Parameter(torch.zeros(hidden, **kw))
        else:
            self.register_parameter("b_g", None)
            self.register_parameter("b_fc", None)
        bound = 1.0 / math.sqrt(in_features)
        with torch.no_grad():
            self.w_g.uniform_(-bound, bound)
            self.w_fc.uniform_(-bound, bound)

    def forward(self, x):
        return swiglu(x, self.w_g, self.w_fc, self.b_g, self.b_fc)
