"""Sum of squares of a row, rounded once to float32.

TEST INFRASTRUCTURE (CPU oracle; see the package docstring for who may use it).

The pages compute ``x.float().pow(2).mean(-1)`` (chapter 13 fusion page,
``torch_reference_fused``; chapter 17 page, the forward kernel's
``reduce_sum``) and leave the order of the fp32 additions open. The one fp32
value of that sum that does not depend on an order is the exact sum rounded
once to fp32, and that is the value this oracle takes.

Squares of bf16/fp16 values are exact in float64 (at most 22 significand
bits), so a float64 sum is exact whenever every partial sum fits in 53 bits.
That is proven per row from the data: if every square is a multiple of 2^L
and the total is below 2^(L+53), every partial sum in any order is exact.
Rows without that proof are summed with Python integers (exact rationals) and
rounded to fp32 by hand.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

__all__ = ["sum_squares_f32", "sum_squares_exact_mask", "fraction_to_f32"]


def _lowest_bit_exponent(v: np.ndarray) -> np.ndarray:
    """For positive finite float64 v, the exponent k of the lowest set bit (v = odd * 2^k)."""
    m, e = np.frexp(v)  # v = m * 2^e, m in [0.5, 1)
    mi = np.ldexp(m, 53).astype(np.uint64)  # exact 53-bit integer significand
    # trailing zeros of mi
    tz = np.zeros(v.shape, dtype=np.int64)
    work = mi.copy()
    for sh in (32, 16, 8, 4, 2, 1):
        mask = np.uint64((1 << sh) - 1)
        z = (work & mask) == 0
        tz += np.where(z, sh, 0)
        work = np.where(z, work >> np.uint64(sh), work)
    return e.astype(np.int64) - 53 + tz


def sum_squares_exact_mask(x32: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float64 row sums of squares and a per-row flag "proven exact"."""
    x64 = np.asarray(x32, dtype=np.float32).astype(np.float64)
    sq = x64 * x64  # exact: the inputs carry at most 11 significand bits
    s64 = sq.sum(axis=-1)
    nz = sq != 0
    big = np.iinfo(np.int64).max
    low = np.where(nz, _lowest_bit_exponent(np.where(nz, sq, 1.0)), big)
    lmin = low.min(axis=-1)
    # total < 2^(L+53)  <=>  every partial sum (any order) is an exact float64
    with np.errstate(over="ignore"):
        limit = np.where(lmin == big, np.inf, np.ldexp(1.0, np.clip(lmin + 53, -1074, 1023)))
    exact = (s64 < limit) | (lmin == big)
    return s64, exact


def fraction_to_f32(q: Fraction) -> np.float32:
    """Round an exact non-negative rational to float32 (nearest, ties to even)."""
    if q < 0:
        raise ValueError("negative")
    if q == 0:
        return np.float32(0.0)
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # normalise so that 2^e <= q < 2^(e+1)
    if (n << max(0, -e)) < (d << max(0, e)):
        e -= 1
    quantum = max(e - 23, -149)  # float32 spacing at this binade (subnormals below 2^-126)
    # m = q / 2^quantum, rounded half to even
    if quantum >= 0:
        num, den = n, d << quantum
    else:
        num, den = n << (-quantum), d
    m, rem = divmod(num, den)
    if 2 * rem > den or (2 * rem == den and (m & 1)):
        m += 1
    val = np.ldexp(np.float64(m), quantum)
    if val > np.finfo(np.float32).max:
        return np.float32(np.inf)
    return np.float32(val)  # exact: m has at most 25 bits and lands on the fp32 grid


def sum_squares_f32(x32: np.ndarray) -> np.ndarray:
    """Per-row exact sum of squares, rounded once to float32. x32: [..., N] float32."""
    x32 = np.asarray(x32, dtype=np.float32)
    s64, exact = sum_squares_exact_mask(x32)
    with np.errstate(over="ignore"):  # (sums past the fp32 range round to infinity, as IEEE prescribes)
        out = s64.astype(np.float32)  # single rounding where the float64 sum is exact
    if not np.all(exact):
        flat_x = x32.reshape(-1, x32.shape[-1])
        flat_out = out.reshape(-1)
        for i in np.flatnonzero(~exact.reshape(-1)):
            tot = sum((Fraction(float(v)) ** 2 for v in flat_x[i]), Fraction(0))
            flat_out[i] = fraction_to_f32(tot)
        out = flat_out.reshape(out.shape)
    return out
