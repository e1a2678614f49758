"""torch.autograd integration of the RMSNorm entry points.

Chapter 17 page ``rmsnorm_tl.py`` wraps its kernels in an autograd Function:
the forward keeps x, w and the per-row rstd, the backward runs the backward
kernel and casts grad_w to the weight dtype. ``RMSNormFunction`` does the same
over ``rnq_rmsnorm_fwd`` / ``rnq_rmsnorm_bwd``; ``RMSNormRoPEFunction`` covers
RMSNorm followed by the partial NeoX RoPE of the chapter 13 fusion page
(``rnq_rmsnorm_rope`` forward, ``rnq_rmsnorm_rope_bwd`` backward: the gradient
through the transposed rotation, then the RMSNorm backward with rstd
recomputed from x). cos/sin are inputs without gradient.

Only GPU tensors are accepted (the entry points raise otherwise); there is no
CPU path.
"""

from __future__ import annotations

import torch

from . import rmsnorm as _rmsnorm
from . import rmsnorm_bwd as _rmsnorm_bwd
from . import rmsnorm_rope as _rmsnorm_rope
from . import rmsnorm_rope_bwd as _rmsnorm_rope_bwd

__all__ = ["RMSNormFunction", "RMSNormRoPEFunction", "rmsnorm", "rmsnorm_rope"]


def _rows(t: torch.Tensor) -> torch.Tensor:
    return t.reshape(-1, t.shape[-1]).contiguous()


class RMSNormFunction(torch.autograd.Function):
    """y = RMSNorm(x, w) over the last dimension; rstd saved for the backward."""

    @staticmethod
    def forward(ctx, x, w, eps=1e-6):
        x2 = _rows(x)
        y, rstd = _rmsnorm(x2, w.contiguous(), eps=eps, return_rstd=True)
        ctx.save_for_backward(x2, w, rstd)
        ctx.eps = eps
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, grad_y):
        x2, w, rstd = ctx.saved_tensors
        gy = _rows(grad_y).to(x2.dtype)
        gx, gw = _rmsnorm_bwd(x2, w.contiguous(), gy, rstd, eps=ctx.eps)
        return (gx.view(grad_y.shape) if ctx.needs_input_grad[0] else None,
                gw.to(w.dtype) if ctx.needs_input_grad[1] else None, None)


class RMSNormRoPEFunction(torch.autograd.Function):
    """y = RoPE_tail(RMSNorm(x, w)); row m of the flattened x uses table row
    m // rows_per_token of cos/sin [T, R/2] (fp32)."""

    @staticmethod
    def forward(ctx, x, w, cos, sin, rows_per_token=1, eps=1e-6):
        x2 = _rows(x)
        cos, sin = cos.contiguous(), sin.contiguous()
        y = _rmsnorm_rope(x2, w.contiguous(), cos, sin, rows_per_token=rows_per_token, eps=eps)
        ctx.save_for_backward(x2, w, cos, sin)
        ctx.rows_per_token = rows_per_token
        ctx.eps = eps
        return y.view(x.shape)

    @staticmethod
    def backward(ctx, grad_y):
        x2, w, cos, sin = ctx.saved_tensors
        gy = _rows(grad_y).to(x2.dtype)
        gx, gw = _rmsnorm_rope_bwd(x2, w.contiguous(), gy, cos, sin, rows_per_token=ctx.rows_per_token, eps=ctx.eps)
        return (gx.view(grad_y.shape) if ctx.needs_input_grad[0] else None,
                gw.to(w.dtype) if ctx.needs_input_grad[1] else None, None, None, None, None)


def rmsnorm(x: torch.Tensor, w: torch.Tensor, eps: float = 1e-6) -> torch.Tensor:
    """Differentiable RMSNorm over the last dimension (the chapter 17 entry point's signature)."""
    return RMSNormFunction.apply(x, w, eps)


def rmsnorm_rope(x: torch.Tensor, w: torch.Tensor, cos: torch.Tensor, sin: torch.Tensor, eps: float = 1e-6,
                 rows_per_token: int | None = None) -> torch.Tensor:
    """Differentiable RMSNorm + RoPE of the last 2 * cos.shape[-1] columns.

    x is [..., D] with D in {64, 128, 256, 512}; cos/sin [T, R/2]. By default
    the flattened rows are split evenly over the T table rows (x [T, H, D]
    gives rows_per_token = H)."""
    if rows_per_token is None:
        rows = x.numel() // x.shape[-1]
        if cos.shape[0] == 0 or rows % cos.shape[0]:
            raise ValueError(f"{rows} rows do not split evenly over {cos.shape[0]} table rows")
        rows_per_token = rows // cos.shape[0]
    return RMSNormRoPEFunction.apply(x, w, cos, sin, rows_per_token, eps)
