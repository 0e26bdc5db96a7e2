"""The exactness arguments the kernels rest on, checked on the CPU in IEEE binary32
(tests/c/div_rn_check.c, built with gcc -ffp-contract=off -fopenmp):

- Markstein's correction step fma(-fma(q0, d, -x), y, q0) with y = fl(1/d),
  q0 = fl(x*y) equals fl(x / d) for every BF16 numerator significand and every
  numerator fl(a * F(1/6)) (a BF16) against every FP32 divisor significand
  (exhaustive: 2^30 and 2^31 pairs), and for arbitrary FP32 numerators on random
  pairs and pairs whose quotient lies next to a rounding midpoint.  The FP8 and
  NVFP4 encoders divide this way; onnxruntime PR #33644 (Description) reports the
  one-ulp differences at E4M3 midpoints that an inexact division causes.
- The NVFP4 scale tables' product multipliers: a multiplier the search accepts at
  the 14 boundary-adjacent BF16 values gives the exact division's E2M1 code for
  every BF16 input, for 512 tensor scales (brute force over all BF16 values).
- The stochastic multipliers: a multiplier the search accepts at the BF16 values next
  to the stochastic rule's grid points gives, for every BF16 input, the same grid
  spacing and floor(256 f) as the exact quotient (so the same code for every random
  byte), for 512 tensor scales."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c", "div_rn_check.c")


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path_factory.mktemp("exact") / "div_rn_check")
    subprocess.run([gcc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off", "-fopenmp", SRC,
                    "-o", exe, "-lm"], check=True, capture_output=True, text=True)
    return exe


def run(exe, *args):
    env = dict(os.environ, OMP_NUM_THREADS=str(min(8, os.cpu_count() or 1)))
    r = subprocess.run([exe, *map(str, args)], env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_markstein_bf16_numerators(checker):
    assert "1073741824 checks, 0 mismatches" in run(checker, "bf16")


def test_markstein_block_scale_numerators(checker):
    assert "2147483648 checks, 0 mismatches" in run(checker, "sixth")


def test_markstein_general_numerators(checker):
    assert "100663296 checks, 0 mismatches" in run(checker, "general", 1 << 24, 0x5EED)


def test_product_multipliers_every_bf16_input(checker):
    out = run(checker, "tables", 512, 0x7AB1E)
    assert " 0 mismatches" in out
    # the search finds a multiplier for most entries and flags the rest (the
    # factor-3 maxima), so both kinds of entry occur
    line = next(l for l in out.splitlines() if l.startswith("tables:") and "without" in l)
    found, without = int(line.split(",")[1].split()[0]), int(line.split(",")[2].split()[0])
    assert found > 100000 and without > 0


def test_stochastic_multipliers_every_bf16_input(checker):
    out = run(checker, "srtables", 512, 0x5A7)
    assert " 0 mismatches" in out
    line = next(l for l in out.splitlines() if l.startswith("srtables:") and "without" in l)
    found, without = int(line.split(",")[1].split()[0]), int(line.split(",")[2].split()[0])
    assert found > 100000 and without > 0


def test_stochastic_grid_points_are_short():
    """The stochastic multiplier criterion compares quotients only down to 9 mantissa
    bits. That is enough because every point where the stochastic rule's reading changes
    (the multiples of D/256 below 6 for grid spacing D = 0.5, 1, 2 below 2, 4, 6, and
    6 itself) is a multiple of 2^(E-9) in its binade [2^E, 2^(E+1))."""
    from fractions import Fraction
    points = set()
    for lo, hi, D in ((0, 2, Fraction(1, 2)), (2, 4, Fraction(1)), (4, 6, Fraction(2))):
        j = 1
        while D * j / 256 < hi:
            if D * j / 256 >= lo:
                points.add(D * j / 256)
            j += 1
    points.add(Fraction(6))
    assert len(points) == 1792
    for g in points:
        E = g.numerator.bit_length() - g.denominator.bit_length()
        if Fraction(2) ** E > g:
            E -= 1
        assert Fraction(2) ** E <= g < Fraction(2) ** (E + 1)
        assert (g / Fraction(2) ** (E - 9)).denominator == 1, g
