"""RMSNorm -> partial NeoX RoPE -> per-row FP8 e4m3fn, row by row, in numpy.

TEST INFRASTRUCTURE (CPU oracle; see the package docstring for who may use it).

Sources (tilelang-tutorial pages):

* chapter 13 fusion page ``rmsnorm_rope_quant.py``: ``torch_reference_fused``
  (RMSNorm in fp32, normalised row cast back to the input dtype, RoPE on the
  last ``rope_dim`` columns, per-row absmax clamped below at 1e-4, scale =
  amax / fp8_max, codes = cast of y / scale) and ``_torch_rope_neox`` (NeoX
  half split: element p pairs with p + rope_dim/2, lo' = lo c - hi s,
  hi' = hi c + lo s, in fp32, cast to the input dtype); the quantising kernel
  clamps y / scale to +-fp8_max before the cast.
* chapter 28 page ``case_norm_rope_quant.py``, module docstring: rows are
  (token, head) pairs normalised over head_dim, every head of a token uses
  the same cos/sin row, one fp32 scale per row.

All arithmetic below is IEEE float32 (numpy evaluates each operation on its
own, rounded to nearest even, with no fused multiply-add), in the order the
reference writes it: ``(x * rstd) * w``, ``(lo*c) - (hi*s)``,
``(hi*c) + (lo*s)``, ``y / scale``. rsqrt is read as 1 / sqrt with both
operations correctly rounded.
"""

from __future__ import annotations

import numpy as np

from .codecs import dtype_round, dtype_to_f32, e4m3_encode
from .exact import sum_squares_f32

__all__ = [
    "rmsnorm_fwd",
    "rope_tail",
    "quantize_rows",
    "norm_rope_quant_rows",
    "qk_norm_rope_fp8",
    "rmsnorm_rope",
    "quantize_groups",
    "rmsnorm_rope_fp8_grouped",
    "truth_norm_rope",
]

F32 = np.float32


def _rstd(x32: np.ndarray, eps: float) -> np.ndarray:
    """rstd = 1 / sqrt(mean(x^2) + eps), every step an fp32 operation."""
    n = x32.shape[-1]
    s = sum_squares_f32(x32)
    ms = s / F32(n)
    v = ms + F32(eps)
    return F32(1.0) / np.sqrt(v)


def rmsnorm_fwd(x_bits: np.ndarray, w_bits: np.ndarray, eps: float, dtype: str = "bf16"):
    """RMSNorm forward. x_bits [M, N], w_bits [N] (uint16 storage of ``dtype``).

    Returns (y_bits [M, N] uint16, rstd [M] float32).
    """
    x = dtype_to_f32(x_bits, dtype)
    w = dtype_to_f32(w_bits, dtype)
    rstd = _rstd(x, eps)
    t = x * rstd[:, None]
    u = t * w[None, :]
    return dtype_round(u, dtype), rstd


def rope_tail(n_bits: np.ndarray, cos: np.ndarray, sin: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """NeoX rotation of the last 2*cos.shape[-1] columns; other columns pass through.

    n_bits [M, N] uint16, cos/sin [M, R/2] float32 (already gathered per row).
    """
    half = cos.shape[-1]
    y_bits = np.array(n_bits, copy=True)
    if half == 0:
        return y_bits
    N = n_bits.shape[-1]
    R = 2 * half
    n = dtype_to_f32(n_bits, dtype)
    lo = n[:, N - R : N - half]
    hi = n[:, N - half :]
    c = np.asarray(cos, dtype=F32)
    s = np.asarray(sin, dtype=F32)
    new_lo = (lo * c) - (hi * s)
    new_hi = (hi * c) + (lo * s)
    y_bits[:, N - R : N - half] = dtype_round(new_lo, dtype)
    y_bits[:, N - half :] = dtype_round(new_hi, dtype)
    return y_bits


def quantize_rows(y_bits: np.ndarray, fp8_max: float, dtype: str = "bf16"):
    """Per-row absmax FP8: returns (codes [M, N] uint8, scale [M] float32)."""
    y = dtype_to_f32(y_bits, dtype)
    amax = np.abs(y).max(axis=-1) if y.shape[-1] else np.zeros(y.shape[0], F32)
    scale = np.maximum(amax, F32(1e-4)) / F32(fp8_max)
    q = y / scale[:, None]
    q = np.minimum(np.maximum(q, -F32(fp8_max)), F32(fp8_max))
    return e4m3_encode(q), scale.astype(F32)


def norm_rope_quant_rows(x_bits, w_bits, cos_rows, sin_rows, eps, fp8_max, dtype="bf16", quant=True):
    """The whole row pipeline on rows that already carry their own cos/sin rows."""
    n_bits, _ = rmsnorm_fwd(x_bits, w_bits, eps, dtype)
    y_bits = rope_tail(n_bits, cos_rows, sin_rows, dtype)
    if not quant:
        return y_bits, None, None
    codes, scale = quantize_rows(y_bits, fp8_max, dtype)
    return y_bits, codes, scale


def qk_norm_rope_fp8(
    q_bits: np.ndarray,
    k_bits: np.ndarray | None,
    wq_bits: np.ndarray,
    wk_bits: np.ndarray | None,
    cos: np.ndarray,
    sin: np.ndarray,
    eps: float = 1e-6,
    fp8_max: float = 448.0,
    dtype: str = "bf16",
    tokens: np.ndarray | None = None,
):
    """QK-norm prologue. q_bits [T, Hq, D], k_bits [T, Hk, D], cos/sin [T_all, R/2].

    ``tokens`` optionally lists which token indices of the table the given rows
    belong to (for sampled parity checks); by default token t uses table row t.
    Returns dict with q_y, q_codes, q_scale [T, Hq], and the same for k.
    """
    out = {}
    for name, xb, wb in (("q", q_bits, wq_bits), ("k", k_bits, wk_bits)):
        if xb is None or xb.shape[1] == 0:
            out[name + "_y"] = None
            out[name + "_codes"] = None
            out[name + "_scale"] = None
            continue
        T, H, D = xb.shape
        t_idx = np.arange(T) if tokens is None else np.asarray(tokens)
        rows = xb.reshape(T * H, D)
        c = np.repeat(np.asarray(cos)[t_idx], H, axis=0)
        s = np.repeat(np.asarray(sin)[t_idx], H, axis=0)
        y, codes, scale = norm_rope_quant_rows(rows, wb, c, s, eps, fp8_max, dtype)
        out[name + "_y"] = y.reshape(T, H, D)
        out[name + "_codes"] = codes.reshape(T, H, D)
        out[name + "_scale"] = scale.reshape(T, H)
    return out


def rmsnorm_rope(x_bits, w_bits, cos, sin, eps=1e-6, dtype="bf16", rows_per_token=1, rows=None):
    """RMSNorm + partial RoPE without quantisation. Row r uses table row r // rows_per_token.

    ``rows`` optionally gives the global row indices of ``x_bits`` (sampled checks).
    """
    M = x_bits.shape[0]
    r = np.arange(M) if rows is None else np.asarray(rows)
    t = r // rows_per_token
    y, _, _ = norm_rope_quant_rows(x_bits, w_bits, np.asarray(cos)[t], np.asarray(sin)[t],
                                   eps, 448.0, dtype, quant=False)
    return y


def quantize_groups(y_bits: np.ndarray, group_size: int, fp8_max: float, dtype: str = "bf16"):
    """Per-group absmax FP8 (chapter 13 fusion page, ``rms_norm_rope_quant_fused``:
    every ``group_size`` consecutive elements of a row share one scale, the
    group's absmax clamped below at 1e-4 over fp8_max; y / scale clamped to
    +-fp8_max, then cast). Returns (codes [M, N] uint8, scale [M, N / group_size] float32).
    """
    y = dtype_to_f32(y_bits, dtype)
    M, N = y.shape
    if N % group_size:
        raise ValueError("group_size must divide the row")
    groups = y.reshape(M, N // group_size, group_size)
    amax = np.abs(groups).max(axis=-1)
    scale = np.maximum(amax, F32(1e-4)) / F32(fp8_max)
    q = groups / scale[:, :, None]
    q = np.minimum(np.maximum(q, -F32(fp8_max)), F32(fp8_max))
    return e4m3_encode(q).reshape(M, N), scale.astype(F32)


def rmsnorm_rope_fp8_grouped(x_bits, w_bits, cos, sin, group_size, eps=1e-6, fp8_max=448.0, dtype="bf16",
                             rows_per_token=1, rows=None):
    """RMSNorm -> partial RoPE -> per-group FP8 over rows of any width (row r uses
    table row r // rows_per_token). Returns (y_bits, codes, scale [M, N / group_size])."""
    y = rmsnorm_rope(x_bits, w_bits, cos, sin, eps, dtype, rows_per_token, rows)
    codes, scale = quantize_groups(y, group_size, fp8_max, dtype)
    return y, codes, scale


def truth_norm_rope(x_bits, w_bits, cos_rows, sin_rows, eps, dtype="bf16", round_intermediates=False):
    """float64 evaluation of RMSNorm + RoPE (the same composition, no fp32 steps).

    With ``round_intermediates`` the two casts to the input dtype are kept
    (applied to the float64 values); without them the result is the exact
    real-arithmetic map, used by the pins that hold only there.
    Returns float64 y [M, N].
    """
    x = dtype_to_f32(x_bits, dtype).astype(np.float64)
    w = dtype_to_f32(w_bits, dtype).astype(np.float64)
    ms = (x * x).mean(axis=-1)
    rstd = 1.0 / np.sqrt(ms + float(np.float32(eps)))
    n = x * rstd[:, None] * w[None, :]

    def rnd(v):
        if not round_intermediates:
            return v
        # float64 -> dtype in one rounding: go through the exact bit pattern
        return _round64_to_dtype(v, dtype)

    n = rnd(n)
    half = cos_rows.shape[-1]
    y = n.copy()
    if half:
        N = x.shape[-1]
        R = 2 * half
        lo = n[:, N - R : N - half]
        hi = n[:, N - half :]
        c = np.asarray(cos_rows, dtype=np.float64)
        s = np.asarray(sin_rows, dtype=np.float64)
        y[:, N - R : N - half] = rnd(lo * c - hi * s)
        y[:, N - half :] = rnd(hi * c + lo * s)
    return y


def _round64_to_dtype(v: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> nearest bf16/fp16 value (ties to even), returned as float64."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "fp16":
        return v.astype(np.float16).astype(np.float64)
    # bf16: 8 significand bits. Scale each value to an integer significand and round half-even.
    out = np.zeros_like(v)
    nz = v != 0
    m, e = np.frexp(v[nz])  # |m| in [0.5, 1)
    e = np.maximum(e, -125)  # bf16 subnormals share the fp32 exponent floor
    q = np.rint(np.ldexp(v[nz], 8 - e))
    out[nz] = np.ldexp(q, e - 8)
    return out
