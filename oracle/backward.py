"""RMSNorm backward in float64.

TEST INFRASTRUCTURE (CPU oracle; see the package docstring for who may use it).

Source: chapter 17 page ``rmsnorm_tl.py``, ``RMSNormTileLang.backward``. With
xn = x * rstd and g = grad_y * w (per row, rstd = 1/sqrt(mean(x^2) + eps)):

    grad_w = sum over rows of grad_y * xn
    grad_x = rstd * (g - xn * mean(g * xn))

The page evaluates this in fp32 torch ops and casts grad_x to the input dtype
and grad_w to the weight dtype; the comparison with the GPU is to a relative
tolerance, so the oracle evaluates the same formula in float64 on the exact
input values and leaves the final casts to the caller.
"""

from __future__ import annotations

import numpy as np

from .codecs import dtype_to_f32

__all__ = ["rmsnorm_bwd"]


def rmsnorm_bwd(x_bits, w_bits, gy_bits, eps: float, dtype: str = "bf16", rstd=None):
    """Returns (grad_x [M, N] float64, grad_w [N] float64, rstd [M] float64).

    ``rstd`` (optional, [M]) replaces the recomputed one, as when the forward
    saved it.
    """
    x = dtype_to_f32(x_bits, dtype).astype(np.float64)
    w = dtype_to_f32(w_bits, dtype).astype(np.float64)
    gy = dtype_to_f32(gy_bits, dtype).astype(np.float64)
    if rstd is None:
        rstd = 1.0 / np.sqrt((x * x).mean(axis=-1) + float(np.float32(eps)))
    else:
        rstd = np.asarray(rstd, dtype=np.float64)
    xn = x * rstd[:, None]
    grad_w = (gy * xn).sum(axis=0)
    g = gy * w[None, :]
    c = (g * xn).mean(axis=-1)
    grad_x = rstd[:, None] * (g - xn * c[:, None])
    return grad_x, grad_w, rstd
