"""Pins of the oracle's codecs against an independent library: torch's CPU casts.

The pages cast with torch (``.to(x.dtype)``, ``.to(torch.float8_e4m3fn)``;
chapter 13 fusion page, ``torch_reference_fused``), so torch's own casts are
the reference behaviour the bit-level codecs must reproduce.
"""

import numpy as np
import pytest
import torch

from oracle import codecs


def _rand_f32(n, seed, lo_exp=-140, hi_exp=127):
    rng = np.random.default_rng(seed)
    mant = rng.integers(0, 1 << 23, n, dtype=np.uint32)
    exp = rng.integers(max(lo_exp + 127, 0), min(hi_exp + 127, 254) + 1, n, dtype=np.uint32)
    sign = rng.integers(0, 2, n, dtype=np.uint32)
    return ((sign << 31) | (exp << 23) | mant).view(np.float32)


def _ties_bf16(n, seed):
    rng = np.random.default_rng(seed)
    hi = rng.integers(0, 0x7F7F, n, dtype=np.uint32)
    low = rng.choice(np.array([0x8000, 0x7FFF, 0x8001, 0x0000, 0xFFFF], dtype=np.uint32), n)
    return ((hi << 16) | low).view(np.float32)


def test_bf16_round_matches_torch():
    x = np.concatenate([_rand_f32(1 << 20, 1), _ties_bf16(1 << 18, 2),
                        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, -1e-45], np.float32)])
    ours = codecs.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    # decode is exact and inverse on the bf16 grid
    assert np.array_equal(codecs.bf16_round(codecs.bf16_to_f32(ours)), ours)


def test_f16_round_matches_torch():
    x = np.concatenate([_rand_f32(1 << 20, 3, -30, 16),
                        np.array([0.0, -0.0, 65504.0, 65520.0 - 1, 2.0**-24, 2.0**-25, 3 * 2.0**-26], np.float32)])
    ours = codecs.f16_round(x)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert list(np.flatnonzero(nan)) == [0x7F, 0xFF]


def _e4m3_probe_values():
    vals = codecs.E4M3_TABLE[np.isfinite(codecs.E4M3_TABLE)]
    pos = np.unique(np.abs(vals))
    mids = (pos[:-1] + pos[1:]) / 2.0  # every rounding boundary (exact in fp32)
    f = np.concatenate([pos, mids]).astype(np.float32)
    u = f.view(np.uint32)
    around = []
    for d in (-2, -1, 1, 2):
        around.append((u.astype(np.int64) + d).clip(0).astype(np.uint32).view(np.float32))
    probe = np.concatenate([f] + around)
    probe = probe[np.abs(probe) <= 448.0]
    rng = np.random.default_rng(7)
    rand = (rng.random(1 << 20) * 2 - 1).astype(np.float32) * 448.0
    small = (rng.random(1 << 18) * 2 - 1).astype(np.float32) * 2.0**-5
    return np.concatenate([probe, -probe, rand, small])


def test_e4m3_encode_matches_torch():
    x = _e4m3_probe_values()
    ours = codecs.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize(
    "value,code",
    [(448.0, 0x7E), (-448.0, 0xFE), (2.0**-9, 0x01), (2.0**-6, 0x08), (1.0, 0x38),
     (-0.0, 0x80), (0.0, 0x00), (2.0**-10, 0x00), (1.5 * 2.0**-10, 0x01), (1.0 + 1 / 16, 0x38),
     (1.0 + 3 / 16, 0x3A), (464.0, 0x7E)],
)
def test_e4m3_special_values(value, code):
    """Values fixed by the format definition (bias 7, 3 mantissa bits, max 448, ties to even)."""
    assert int(codecs.e4m3_encode(np.float32(value))) == code


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        codecs.e4m3_encode(np.float32(465.0))
