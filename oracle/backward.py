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

__all__ = ["rmsnorm_bwd", "rope_bwd_rotate", "rmsnorm_rope_bwd"]


def _bwd_f64(x, w, gy, eps, rstd):
    """The chapter 17 backward on float64 arrays: (grad_x, grad_w, rstd)."""
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


def rmsnorm_bwd(x_bits, w_bits, gy_bits, eps: float, dtype: str = "bf16", rstd=None):
    """Returns (grad_x [M, N] float64, grad_w [N] float64, rstd [M] float64).

    ``rstd`` (optional, [M]) replaces the recomputed one, as when the forward
    saved it.
    """
    x = dtype_to_f32(x_bits, dtype).astype(np.float64)
    w = dtype_to_f32(w_bits, dtype).astype(np.float64)
    gy = dtype_to_f32(gy_bits, dtype).astype(np.float64)
    return _bwd_f64(x, w, gy, eps, rstd)


def rope_bwd_rotate(gy, cos_rows, sin_rows):
    """Gradient through the NeoX rotation of the last R = 2 * half columns.

    The forward (chapter 13 fusion page, the rotate-half RoPE of the normalised
    tail) maps a pair (lo, hi) = (n[p], n[p + half]) of the tail to
    (lo c - hi s, hi c + lo s): multiplication by the rotation matrix
    [[c, -s], [s, c]]. Its vector-Jacobian product is multiplication by the
    transpose, (g_lo c + g_hi s, g_hi c - g_lo s). Columns before the tail
    pass their gradient through unchanged. float64 in, float64 out.
    """
    g = np.array(gy, dtype=np.float64, copy=True)
    half = np.asarray(cos_rows).shape[-1]
    if half == 0:
        return g
    N = g.shape[-1]
    c = np.asarray(cos_rows, dtype=np.float64)
    s = np.asarray(sin_rows, dtype=np.float64)
    lo = g[:, N - 2 * half : N - half].copy()
    hi = g[:, N - half :].copy()
    g[:, N - 2 * half : N - half] = lo * c + hi * s
    g[:, N - half :] = hi * c - lo * s
    return g


def rmsnorm_rope_bwd(x_bits, w_bits, gy_bits, cos, sin, eps: float, dtype: str = "bf16", rows_per_token: int = 1,
                     rstd=None):
    """Backward of RMSNorm followed by the partial RoPE of the last R columns.

    Differentiates the real-valued map (the two casts to the input dtype taken
    as identities, as the chapter 17 backward does for its own cast): the
    output gradient goes back through the rotation (``rope_bwd_rotate``, table
    row r // rows_per_token for row r), then through the chapter 17 RMSNorm
    backward. Returns (grad_x [M, N] float64, grad_w [N] float64, rstd [M]).
    """
    x = dtype_to_f32(x_bits, dtype).astype(np.float64)
    w = dtype_to_f32(w_bits, dtype).astype(np.float64)
    gy = dtype_to_f32(gy_bits, dtype).astype(np.float64)
    t = np.arange(x.shape[0]) // rows_per_token
    gn = rope_bwd_rotate(gy, np.asarray(cos)[t], np.asarray(sin)[t])
    return _bwd_f64(x, w, gn, eps, rstd)
