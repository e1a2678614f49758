"""Rows that put FP8 quotients exactly on e4m3 rounding midpoints.

Test input construction only (exact rational arithmetic, no step of the
method): an e4m3 code flips there with one rounding more or less, so these rows
separate a correctly rounded y / scale from any cheaper approximation.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from oracle import codecs

_ODD = {448.0: 7, 240.0: 15}  # odd part of fp8_max


def e4m3_midpoints() -> list[Fraction]:
    """Every point halfway between two neighbouring finite e4m3fn magnitudes."""
    v = np.unique(np.abs(codecs.e4m3_decode(np.arange(256, dtype=np.uint8)).astype(np.float64)))
    v = v[np.isfinite(v)]
    return [(Fraction(float(a)) + Fraction(float(b))) / 2 for a, b in zip(v[:-1], v[1:])]


def _is_bf16(f: float) -> bool:
    return float(codecs.bf16_to_f32(codecs.bf16_round(np.float32(f)))) == f


def tie_values(fp8_max: float, amax: Fraction) -> list[float]:
    """bf16 values y (both signs) with y * fp8_max / amax an e4m3 midpoint."""
    out = []
    for m in e4m3_midpoints():
        if m >= Fraction(fp8_max):
            break  # (|y| <= amax keeps |y / scale| <= fp8_max)
        y = m * amax / Fraction(fp8_max)
        if _is_bf16(float(y)) and Fraction(float(y)) == y:
            out += [float(y), -float(y)]
    return out


def tie_rows(fp8_max: float, exps=(-6, 0, 3), width: int = 128) -> np.ndarray:
    """bf16 bits [rows, width]: column 0 is amax (an odd significand divisible
    by fp8_max's odd part, times 2^e), the others tie values of that amax (zero
    where a row runs out of them)."""
    odd = _ODD[fp8_max]
    rows = []
    for a_odd in range(odd, 256, 2 * odd):
        for e in exps:
            amax = Fraction(a_odd) * Fraction(2) ** e
            ys = tie_values(fp8_max, amax)
            for i in range(0, len(ys), width - 1):
                row = np.zeros(width, np.float32)
                row[0] = float(amax)
                chunk = ys[i:i + width - 1]
                row[1:1 + len(chunk)] = chunk
                rows.append(row)
    return codecs.bf16_round(np.stack(rows))


def _largest_bf16_square_at_most(d: Fraction, cap: Fraction, quantum: Fraction) -> Fraction:
    """The largest bf16 multiple f of ``quantum`` with f <= cap and f^2 <= d."""
    f = float(min(cap, Fraction(np.sqrt(float(d)))))
    b = codecs.bf16_round(np.float32(f))
    while True:
        v = Fraction(float(codecs.bf16_to_f32(b)))
        if v <= cap and v * v <= d and (v / quantum).denominator == 1:
            return v
        b = np.uint16(int(b) - 1)


def _lowest_bit(q: Fraction) -> int:
    """k with q = odd * 2^k (q > 0 dyadic)."""
    n, d = q.numerator, q.denominator
    return (n & -n).bit_length() - 1 - (d.bit_length() - 1)


def normalised_tie_rows(fp8_max: float, width: int = 128, ties_per_row: int = 16):
    """Rows whose RMSNorm (eps = 0, w = 1) is the identity: column 0 amax, then up
    to ``ties_per_row`` tie values, then filler values (each at most amax) that
    bring the sum of squares to exactly ``width``, so mean(x^2) = 1, rstd = 1 and
    the normalised row is the row itself (also when rows are laid side by side
    into a wider row). amax is scaled by a power of two into [1.13, 2.26): with
    16 ties the sum is then at most 17 amax^2 < width, and the rest fits the
    filler columns (including the few the greedy completion spends on low bits).
    Returns bf16 bits [rows, width]."""
    odd = _ODD[fp8_max]
    rows = []
    for a_odd in range(odd, 256, 2 * odd):
        amax = Fraction(a_odd)
        while amax >= Fraction(226, 100):
            amax /= 2
        while amax < Fraction(113, 100):
            amax *= 2
        # largest first, so that each row's values span as few binades as possible
        ys = sorted(tie_values(fp8_max, amax), key=abs, reverse=True)
        for i in range(0, len(ys), ties_per_row):
            vals = [amax] + [Fraction(y) for y in ys[i:i + ties_per_row]]
            d = Fraction(width) - sum(v * v for v in vals)
            fill = []
            if d > 0:
                # fillers are multiples of 2^floor(L/2), L the lowest bit of d: their
                # squares add no bit below those already there
                quantum = Fraction(2) ** (_lowest_bit(d) // 2)
                while d > 0 and len(vals) + len(fill) < width:
                    f = _largest_bf16_square_at_most(d, amax, quantum)
                    fill.append(f)
                    d -= f * f
            if d != 0:
                raise AssertionError(f"no exact completion for amax {amax}")
            row = np.zeros(width, np.float32)
            allv = vals + fill
            row[: len(allv)] = [float(v) for v in allv]
            rows.append(row)
    return codecs.bf16_round(np.stack(rows))


def lowest_square_bit(bits: np.ndarray) -> np.ndarray:
    """Per row of bf16 bits: the exponent of the lowest set bit over the squares
    of its nonzero values (a float64 sum of the squares is exact in any order
    while the total stays below 2^(that + 53))."""
    vals = codecs.bf16_to_f32(bits)
    out = []
    for row in vals:
        low = [2 * _lowest_bit(abs(Fraction(float(v)))) for v in row if v != 0]
        out.append(min(low) if low else 0)
    return np.array(out)

