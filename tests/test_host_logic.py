"""Host-side decisions of the launchers, checked on the CPU (no GPU use):

* row -> token by multiply-shift (exact for every row below 2^31);
* whether quotients are clamped to +-fp8_max before encoding: needed exactly
  when some fp32 value between fp8_max and fp8_max * (1 + 2^-20) (a margin
  above the largest quotient |y / scale| can reach) encodes to another e4m3
  code than fp8_max itself (encoder: the oracle's, pinned against torch);
* the row kernel's pass layout (which kernel variant a launch takes), against
  its definition restated here, at the limits of each condition.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from oracle import codecs

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bin", "host_logic_check")


def _exe():
    if not os.path.exists(EXE):
        pytest.skip("host_logic_check not built (python -m fp8_quant_amd.build)")
    return EXE


def test_row_to_token_division_is_exact():
    out = subprocess.run([_exe(), "div"], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stdout + out.stderr
    assert ", 0 wrong" in out.stdout


def _clamp_needed_definition(f: float) -> bool:
    f32 = np.float32(f)
    hi = np.float32(np.float64(f32) * (1 + 2.0**-20))
    vals = np.arange(f32.view(np.uint32), hi.view(np.uint32) + 1, dtype=np.uint32).view(np.float32)
    codes = codecs.e4m3_encode(vals)
    return bool((codes != codes[0]).any())


def _candidates():
    # every positive e4m3 value below 448, the midpoints between neighbours and the
    # fp32 values just around them, plus a few round numbers
    dec = codecs.e4m3_decode(np.arange(1, 0x7F, dtype=np.uint8)).astype(np.float64)
    dec = np.unique(dec[dec > 0])
    mids = (dec[:-1] + dec[1:]) / 2
    out = set()
    for m in np.r_[dec, mids]:
        m32 = np.float32(m)
        for v in (np.nextafter(m32, np.float32(0)), m32, np.nextafter(m32, np.float32(np.inf))):
            if 0 < v <= 448:
                out.add(float(v))
    out |= {448.0, 240.0, 57.5, 0.5, 1.0, 1e-3, 3.0, 100.0}
    return sorted(out)


def test_clamp_decision_matches_its_definition():
    fs = _candidates()
    out = subprocess.run([_exe(), "clamp", *[repr(f) for f in fs]], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    got = {}
    for line in out.stdout.split("\n"):
        if line.strip():
            a, b = line.split()
            got[float(a)] = b == "1"
    assert len(got) == len(fs)
    wrong = [f for f in fs if got[f] != _clamp_needed_definition(f)]
    assert not wrong, f"clamp decision differs for fp8_max in {wrong[:10]}"
    # the decision matters somewhere: just below a midpoint the clamp is needed
    assert any(got.values()) and not all(got.values())


# ----------------------------------------------------------------- pass layout

PER_LANE, ONE_TOKEN, WHOLE_TOKENS = 0, 1, 2


def _layout_definition(G, heads, heads0, rows, xs0, D, rope, pos, max_pos):
    """Passes inside one token (both head counts multiples of G); else passes of
    whole tokens of one tensor when the heads per token divide G, the rows fill
    whole passes, a pass's input rows span less than 2^31 bytes with the token
    stride below 2^30 elements, and a position-indexed table stays below 2^31
    bytes; else one row per lane. Returns (layout, log2 of the heads per token)."""
    if heads % G == 0 and heads0 % G == 0:
        return ONE_TOKEN, -1
    if heads0 != heads or G % heads or rows % G:
        return PER_LANE, -1
    shift = (heads - 1).bit_length()
    tokens_per_pass = G // heads
    span = 2 * ((tokens_per_pass - 1) * xs0 + heads * D)
    if span >= 2**31 or xs0 >= 2**30 or (pos and max_pos * (rope // 2) * 4 >= 2**31):
        return PER_LANE, -1
    return WHOLE_TOKENS, shift


def _layout_cases():
    cases = []
    for D in (64, 128, 256, 512):
        G = 64 // (D // 16)
        for heads in (1, 2, 3, 4, 5, 8, 16, 32, 40):
            for heads0 in {heads, max(heads - 1, 1), heads // 2 or 1}:
                for rows in (G * heads * 3, G * heads * 3 + 1):
                    xs_contig = heads0 * D
                    for xs0 in (xs_contig, xs_contig + 8):
                        for rope, pos, max_pos in ((0, 0, 0), (D, 0, 0), (D, 1, 4096)):
                            cases.append((G, heads, heads0, rows, xs0, D, rope, pos, max_pos))
    # the limits: a pass's span at and just below 2^31 bytes, the token stride at
    # 2^30 elements, and a table exactly at and just below 2^31 bytes
    for D, heads in ((128, 1), (128, 2), (64, 4)):
        G = 64 // (D // 16)
        tpp = G // heads
        rows = G * 4
        for span in (2**31 - 2, 2**31):
            xs0 = (span // 2 - heads * D) // (tpp - 1)
            cases.append((G, heads, heads, rows, xs0, D, 0, 0, 0))
            cases.append((G, heads, heads, rows, xs0 + 1, D, 0, 0, 0))
        cases.append((G, heads, heads, rows, 2**30, D, 0, 0, 0))
        cases.append((G, heads, heads, rows, 2**30 - 8, D, 0, 0, 0))
        for rope in (16, 64, D):
            limit = 2**31 // (4 * (rope // 2))
            for max_pos in (limit - 1, limit, limit + 1):
                cases.append((G, heads, heads, rows, heads * D, D, rope, 1, max_pos))
                cases.append((G, heads, heads, rows, heads * D, D, rope, 0, max_pos))
    return cases


def test_row_kernel_pass_layout_matches_its_definition():
    cases = _layout_cases()
    inp = "".join(" ".join(str(v) for v in c) + "\n" for c in cases)
    out = subprocess.run([_exe(), "layout"], input=inp, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    got = [tuple(int(v) for v in line.split()) for line in out.stdout.splitlines()]
    assert len(got) == len(cases)
    bad = [(c, g, _layout_definition(*c)) for c, g in zip(cases, got) if g != _layout_definition(*c)]
    assert not bad, bad[:5]
    kinds = {g[0] for g in got}
    assert kinds == {PER_LANE, ONE_TOKEN, WHOLE_TOKENS}
