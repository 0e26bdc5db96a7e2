"""The oracle's format encoders over every FP32 input: BF16 rounding, E4M3
(saturating, OCP E4M3FN), E2M1 nearest-even and E2M1 stochastic rounding, each
against an independent restatement of the format in integer arithmetic on the bit
pattern (tests/c/oracle_encoders_all_fp32.c, compiled with the oracle's C source,
OpenMP over the 2^32 patterns: about 45 s on 8 cores).  onnxruntime PR #33644
(Description) names the saturating nearest-even E4M3FN encode; the E2M1 grid and the
stochastic rule are the NVFP4 readings O17 and O21."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_encoders_every_fp32_input(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_encoders_all_fp32")
    subprocess.run([gcc, "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off", "-fno-fast-math",
                    "-fopenmp", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "c", "oracle_encoders_all_fp32.c"),
                    os.path.join(ROOT, "oracle", "mxq_oracle.c"), "-o", exe, "-lm"],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS=str(min(16, os.cpu_count() or 1)))
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout + r.stderr
    for name in ("bf16", "e4m3", "e2m1", "e2m1_sr"):
        assert f"{name}: 4294967296 inputs, 0 mismatches" in r.stdout, r.stdout
