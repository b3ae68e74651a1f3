"""The quantizer's per-element quotient, proved by exhaustion on the host.

The GPU quantizer replaces the correctly rounded division x / scale by Markstein's FMA
correction of a reciprocal product. tests/exhaustive/quotient_codes.c runs every (amax, x) pair
the quantizer can meet with a normal scale (531,921,744 pairs) and checks that both quotients
give the same OCP E4M3 code. It uses the C library's fmaf (a correctly rounded fused
multiply-add) and needs no GPU; about 20 s.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "exhaustive", "quotient_codes.c")


def test_fast_quotient_gives_the_division_codes(tmp_path):
    exe = str(tmp_path / "quotient_codes")
    build = subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-o", exe, SRC, "-lm"],
                           capture_output=True, text=True)
    if build.returncode != 0:
        pytest.fail("gcc failed: " + build.stderr[-2000:])
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "code mismatches 0" in run.stdout
    assert "pairs 531921744" in run.stdout
