"""Exhaustive host check behind the binary32-scale blockwise FP8 encoder's
division-free quotient (csrc/quant_mxfp8.hip, f32s_quotient): for every
positive finite BF16 block maximum a whose scale s = RN32(a / 448) is at
least 2^-80, and every BF16 x with |x| <= a (both signs, -0 included), the
signed saturating E4M3 RNE code of the correctly rounded quotient
RN32(x / s) equals that of copysign(fma(fma(-q0, s, x), r, q0), x) with
r = RN32(1 / s) and q0 = RN32(x r).  A fact of IEEE binary32 arithmetic over
a finite domain, checked in C with SSE float division and fmaf (about 1e9
pairs, about a minute)."""

import os
import shutil
import subprocess
import tempfile

import pytest

SRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "exhaustive", "fp8bw_f32_quotient.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_division_free_quotient_gives_the_same_e4m3_codes():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "q")
        subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", exe, SRC, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout
    assert "code mismatches 0" in out.stdout
