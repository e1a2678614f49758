"""Host-side decisions of the launchers, checked on the CPU (no GPU use):

* row -> token by multiply-shift (exact for every row below 2^31);
* whether quotients are clamped to +-fp8_max before encoding: needed exactly
  when some fp32 value between fp8_max and fp8_max * (1 + 2^-20) (a margin
  above the largest quotient |y / scale| can reach) encodes to another e4m3
  code than fp8_max itself (encoder: the oracle's, pinned against torch).
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
