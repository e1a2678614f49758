"""The FP8 step divides y by the row scale with a reciprocal and one FMA
correction instead of a full IEEE division. This checks, on the host, that the
sequence gives the IEEE quotient for every bf16 / fp16 numerator significand
against divisor significands spread over the whole fp32 significand range
(the sequence is exact under power-of-two scaling, so one exponent pair stands
for all normal ranges). A full sweep of all 2^23 divisor significands runs
with RNQ_FULL_QUOTIENT_CHECK=1 (a few seconds per case on 8 cores).
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    cc = shutil.which("gcc")
    if cc is None:
        pytest.skip("gcc not available")
    exe = tmp_path_factory.mktemp("qc") / "quotient_check"
    subprocess.run([cc, "-O2", "-ffp-contract=off", "-march=x86-64-v3", os.path.join(HERE, "csrc", "quotient_check.c"),
                    "-o", str(exe), "-lm"], check=True)
    return str(exe)


@pytest.mark.parametrize("mbits,aexp,bexp", [(7, 0, 0), (7, 5, -9), (7, -20, -30), (10, 0, 0), (10, -3, 4)])
def test_quotient_sequence_matches_ieee_division(checker, mbits, aexp, bexp):
    full = os.environ.get("RNQ_FULL_QUOTIENT_CHECK") == "1"
    step = 1 if full else 257  # every 257th significand: 32k divisors, plus the edges below
    out = subprocess.run([checker, str(mbits), str(aexp), str(bexp), "0", str(1 << 23), str(step)],
                         check=True, capture_output=True, text=True).stdout.split()
    total, bad = int(out[0]), int(out[1])
    assert total > 0 and bad == 0
    # significands next to the binade edges
    for lo, hi in ((0, 4096), ((1 << 23) - 4096, 1 << 23)):
        out = subprocess.run([checker, str(mbits), str(aexp), str(bexp), str(lo), str(hi), "1"],
                             check=True, capture_output=True, text=True).stdout.split()
        assert int(out[1]) == 0
