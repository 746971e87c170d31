"""Exhaustive host proof of the per-token quantiser's division (no GPU).

The quantiser's codes are rint(RN(x / s)) clamped to [-127, 127] with
s = RN(amax / 127) (w8a8_dynamic step, xLLM pull request #1890 review thread;
the symmetric per-row reading).  For rows with amax >= 2^-60 the kernel
replaces the per-element division with one reciprocal per row and Markstein's
correction step.  tests/quant_divide_exhaustive.c replays that fp32 arithmetic
for every positive finite bf16 amax and every bf16 x with |x| <= amax, both
signs (about 1e9 pairs), and compares each code with the correctly rounded
quotient's.  What holds is that every CODE is exact: the corrected quotient
itself differs from RN(x / s) on 1,430,134 pairs, all with |x / s| < 1/4,
where the code is 0 either way.
"""
import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "quant_divide_exhaustive.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path_factory.mktemp("qde") / "quant_divide_exhaustive")
    subprocess.run([gcc, "-O2", "-ffp-contract=off", "-fopenmp", SRC, "-o", exe, "-lm"], check=True)
    return exe


def run(exe, mode):
    out = subprocess.run([exe, str(mode)], check=True, capture_output=True, text=True, timeout=600).stdout
    return {k: int(v) for k, v in re.findall(r"(\w+)=(-?\d+)", out)}


def test_every_code_of_the_fast_division_is_exact(checker):
    r = run(checker, 0)
    # every positive bf16 amax >= 2^-60 with every bf16 |x| <= amax, both signs (x = 0 once)
    assert r["pairs_fast"] == 991_821_824
    assert r["code_mismatch"] == 0
    # the quotient can differ from RN(x / s) only where the code is 0 either way
    assert r["quot_mismatch_ge_quarter"] == 0
    assert r["quot_mismatch"] == 1_430_134
    # |rint(RN(x / s))| <= 127 everywhere, including the rows that divide element by element
    assert r["pairs_slow"] > 0 and r["clamp_binds"] == 0


def test_planted_uncorrected_quotient_is_caught(checker):
    """Without the correction step (q0 = RN(x * RN(1/s)) alone) codes go wrong: the harness sees it."""
    r = run(checker, 1)
    assert r["code_mismatch"] > 0
