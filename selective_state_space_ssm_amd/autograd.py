"""torch.autograd wrappers over the C ABI: the forward keeps only the chunk
states (ssm_scan_fwd_states / ssm_scan_fwd_conv with ``state_chunk``), the
backward recomputes from them (ssm_scan_bwd / ssm_scan_bwd_conv).  Argument
marshalling only; every step runs in the library's kernels.

    y, last_state = selective_scan(u, delta, A, B, C, D, z, delta_bias,
                                   delta_softplus=True, h0=None, state_chunk=128)
    y, last_state = selective_scan_conv(x, conv_w, conv_b, delta, A, B, C, D, z, ...)
    out = out_proj(y, W)          # the Linear after the gate, [b, L, d_model]

Gradients flow to every tensor argument that requires them (dB and dC are
computed in float32 and returned in the dtype of B and C).
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (ssm_out_proj, ssm_out_proj_bwd, ssm_scan_bwd, ssm_scan_bwd_conv, ssm_scan_fwd_conv,
               ssm_scan_fwd_states)

__all__ = ["selective_scan", "selective_scan_conv", "out_proj"]


def _grad_or_zero(g, like):
    return torch.zeros_like(like) if g is None else g.contiguous()


class _SelectiveScan(torch.autograd.Function):
    @staticmethod
    def forward(ctx, u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, state_chunk):
        y, last, cs = ssm_scan_fwd_states(u, delta, A, B, C, D, z, delta_bias, delta_softplus=delta_softplus,
                                          h0=h0, state_chunk=state_chunk)
        ctx.save_for_backward(u, delta, A, B, C, D, z, delta_bias, h0, cs)
        ctx.delta_softplus = delta_softplus
        ctx.state_chunk = state_chunk
        return y, last

    @staticmethod
    def backward(ctx, dy, dlast):
        u, delta, A, B, C, D, z, delta_bias, h0, cs = ctx.saved_tensors
        g = ssm_scan_bwd(u, delta, A, B, C, cs, ctx.state_chunk, _grad_or_zero(dy, u), D=D, z=z,
                         delta_bias=delta_bias, delta_softplus=ctx.delta_softplus, h0=h0,
                         dlast=None if dlast is None else dlast.contiguous(),
                         want_dD=D is not None, want_ddelta_bias=delta_bias is not None, want_dh0=h0 is not None)
        return (g["du"], g["ddelta"], g["dA"], g["dB"].to(B.dtype), g["dC"].to(C.dtype), g["dD"], g["dz"],
                g["ddelta_bias"], g["dh0"], None, None)


def selective_scan(u: torch.Tensor, delta: torch.Tensor, A: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                   D: Optional[torch.Tensor] = None, z: Optional[torch.Tensor] = None,
                   delta_bias: Optional[torch.Tensor] = None, delta_softplus: bool = False,
                   h0: Optional[torch.Tensor] = None, state_chunk: int = 128):
    """Differentiable selective scan: returns (y, last_state)."""
    return _SelectiveScan.apply(u, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, state_chunk)


class _SelectiveScanConv(torch.autograd.Function):
    @staticmethod
    def forward(ctx, x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, delta_softplus, state_chunk):
        y, last, cs, _ = ssm_scan_fwd_conv(x, conv_w, delta, A, B, C, conv_b=conv_b, D=D, z=z,
                                           delta_bias=delta_bias, delta_softplus=delta_softplus, h0=h0,
                                           state_chunk=state_chunk)
        ctx.save_for_backward(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, cs)
        ctx.delta_softplus = delta_softplus
        ctx.state_chunk = state_chunk
        return y, last

    @staticmethod
    def backward(ctx, dy, dlast):
        x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, cs = ctx.saved_tensors
        g = ssm_scan_bwd_conv(x, conv_w, delta, A, B, C, cs, ctx.state_chunk, _grad_or_zero(dy, x), conv_b=conv_b,
                              D=D, z=z, delta_bias=delta_bias, delta_softplus=ctx.delta_softplus, h0=h0,
                              dlast=None if dlast is None else dlast.contiguous())
        return (g["dx"], g["dconv_w"], g["dconv_b"], g["ddelta"], g["dA"], g["dB"].to(B.dtype), g["dC"].to(C.dtype),
                g["dD"] if D is not None else None, g["dz"], g["ddelta_bias"] if delta_bias is not None else None,
                g["dh0"] if h0 is not None else None, None, None)


def selective_scan_conv(x: torch.Tensor, conv_w: torch.Tensor, conv_b: Optional[torch.Tensor], delta: torch.Tensor,
                        A: torch.Tensor, B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None,
                        z: Optional[torch.Tensor] = None, delta_bias: Optional[torch.Tensor] = None,
                        delta_softplus: bool = False, h0: Optional[torch.Tensor] = None, state_chunk: int = 128):
    """Differentiable selective scan with the causal conv1d + SiLU in front
    (u = silu(conv1d(x))): returns (y, last_state)."""
    return _SelectiveScanConv.apply(x, conv_w, conv_b, delta, A, B, C, D, z, delta_bias, h0, delta_softplus,
                                    state_chunk)


class _OutProj(torch.autograd.Function):
    @staticmethod
    def forward(ctx, y, W):
        ctx.save_for_backward(y, W)
        return ssm_out_proj(y, W)

    @staticmethod
    def backward(ctx, dout):
        y, W = ctx.saved_tensors
        dy, dW = ssm_out_proj_bwd(y, W, dout.contiguous(), want_dy=ctx.needs_input_grad[0],
                                  want_dW=ctx.needs_input_grad[1])
        return dy, dW


def out_proj(y: torch.Tensor, W: torch.Tensor) -> torch.Tensor:
    """Differentiable output projection: out[b, t, m] = sum_k W[m, k] y[b, k, t]
    (y [b, d_inner, L] as the scan writes it, W [d_model, d_inner]); returns
    [b, L, d_model]."""
    return _OutProj.apply(y, W)
