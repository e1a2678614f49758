"""Bit-level codecs of the oracle: bfloat16, float16 and OCP float8 e4m3fn.

TEST INFRASTRUCTURE (CPU oracle; see the package docstring for who may use it).

The pages cast with PyTorch (``.to(x.dtype)`` for the bf16/fp16 roundings and
``.to(torch.float8_e4m3fn)`` for the codes, chapter 13 fusion page,
``torch_reference_fused``). Those casts round to nearest, ties to even. The
codecs below restate that rounding from the formats' definitions:

* bfloat16: the upper 16 bits of an IEEE binary32; rounding keeps 8
  significand bits.
* float16: IEEE binary16; numpy's float32 -> float16 conversion is the
  IEEE round-to-nearest-even operation and is used as a library step.
* float8 e4m3fn (OCP 8-bit FP, "fn" = finite, no infinities): 1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds
  subnormals m * 2^-9; the largest finite value is 1.75 * 2^8 = 448
  (code 0x7E); 0x7F / 0xFF are NaN.

Only finite inputs are handled.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_round",
    "bf16_to_f32",
    "f16_round",
    "f16_to_f32",
    "e4m3_encode",
    "e4m3_decode",
    "E4M3_TABLE",
    "dtype_round",
    "dtype_to_f32",
]


def bf16_round(x) -> np.ndarray:
    """float32 -> bfloat16 bits (uint16), round to nearest, ties to even."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_to_f32(b) -> np.ndarray:
    """bfloat16 bits -> float32 (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f16_round(x) -> np.ndarray:
    """float32 -> float16 bits (uint16), IEEE round to nearest even (values past
    the fp16 range become infinities, as IEEE rounding prescribes)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_to_f32(b) -> np.ndarray:
    """float16 bits -> float32 (exact)."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float32)


def dtype_round(x, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "fp16":
        return f16_round(x)
    raise ValueError(dtype)


def dtype_to_f32(b, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f32(b)
    if dtype == "fp16":
        return f16_to_f32(b)
    raise ValueError(dtype)


def _build_e4m3_table() -> np.ndarray:
    """Value of each of the 256 e4m3fn codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = sign * m * 2.0**-9
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_TABLE = _build_e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float32 values."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x) -> np.ndarray:
    """float32 -> e4m3fn codes (uint8), round to nearest, ties to even.

    Inputs must satisfy |x| <= 464 (the callers clamp to +-fp8_max <= 448
    first); zero keeps its sign (-0.0 -> 0x80).
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x).astype(np.float64)
    if np.any(a > 464.0) or np.any(~np.isfinite(a)):
        raise ValueError("e4m3_encode: magnitude beyond the e4m3fn range")
    code = np.zeros(a.shape, dtype=np.int64)

    sub = a < 2.0**-6
    # subnormal range: value = m * 2^-9, m in 0..7; m == 8 is the smallest normal (code 0x08)
    code[sub] = np.rint(a[sub] * 2.0**9).astype(np.int64)

    nrm = ~sub
    if np.any(nrm):
        an = a[nrm]
        _, ex = np.frexp(an)  # an = f * 2^ex with f in [0.5, 1)
        e = ex.astype(np.int64) - 1  # an in [2^e, 2^(e+1))
        mant = np.rint((an / np.exp2(e) - 1.0) * 8.0).astype(np.int64)
        carry = mant == 8
        e = e + carry
        mant = np.where(carry, 0, mant)
        code[nrm] = ((e + 7) << 3) | mant
    code = code | np.where(np.signbit(x), 0x80, 0)
    return code.astype(np.uint8)
