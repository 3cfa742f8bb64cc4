"""The quantizers' per-element division, replayed on the CPU for every pair
of BF16 (x, amax) with |x| <= amax (tests/native/div_check.c).

The 1x128 quantizers compute fl32(x / s) with s = fl32(amax / 448) (page 1,
the uniondaocoop.com post: one scale per 1x128 tile from the tile's maximum
magnitude) without dividing per element: one reciprocal per tile, a product
and one fused correction step, with tiles below 2^-60 evaluated on operands
scaled by 2^64.  The C program repeats those IEEE binary32 operations and
compares them with the correctly rounded quotient over all 2.1e9 pairs,
with and without power-of-two scales.
"""

import os
import re
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "native", "div_check.c")


def build(tmp_path, *defines):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "div_check")
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", *defines, "-o", exe, SRC, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return exe


def run(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    m = re.search(r"pairs (\d+) bit-equal (\d+) both-encode-to-zero (\d+) failures (\d+)", r.stdout)
    assert m, r.stdout + r.stderr
    return r.returncode, [int(v) for v in m.groups()]


def test_corrected_divide_matches_ieee_quotient_for_every_bf16_pair(tmp_path):
    rc, (pairs, equal, zero, fails) = run(build(tmp_path))
    # amax over the 32639 positive finite BF16 values, x over every BF16 of
    # magnitude <= amax with both signs (+-0 included), two scale rules
    assert pairs == 2 * sum(2 * (ab + 1) for ab in range(1, 0x7F80))
    assert fails == 0 and rc == 0
    assert equal > 0.999 * pairs and zero > 0


def test_planted_mistake_is_caught(tmp_path):
    # without the correction step the product x * RN(1/s) is off by an ulp
    # for many pairs: the check must fail
    rc, (_, _, _, fails) = run(build(tmp_path, "-DPLANT_NO_CORRECTION"))
    assert rc != 0 and fails > 1000
