"""The row kernel's fast reciprocal and square root (used inside wave-uniform
range checks, with IEEE fallbacks outside) equal the IEEE results bit for bit
over every positive normal fp32 input, on the GPU itself.
"""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bin", "row_scalar_check")


def test_fast_row_scalars_are_ieee_exact_in_their_ranges():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} not built (run __graft_entry__.build())")
    out = subprocess.run([EXE], check=True, capture_output=True, text=True, timeout=120).stdout
    vals = dict(line.split() for line in out.strip().splitlines())
    print(out, flush=True)
    assert int(vals["rcp_mismatch_in_range"]) == 0
    assert int(vals["sqrt_mismatch_in_range"]) == 0
