"""include/mxq.h from C and C++: a C11 program calls every entry point through the
header's prototypes and types (gcc -std=c11 -Wall -Wextra -Werror -pedantic, linked
against libmxq.so) and checks the host-side answers -- version and status strings,
the workspace-size queries, argument errors of each call -- and a C++17 file takes
the entry points' addresses as pointers to C functions of the declared types.  The
program runs with no GPU visible (HIP_VISIBLE_DEVICES and ROCR_VISIBLE_DEVICES
empty): these paths enqueue nothing, and a check that wrongly accepted a call would
fail its launch instead of touching a device."""
import os
import shutil
import subprocess

import pytest

import nvfp4_quantization_amd as mxq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c")
INC = os.path.join(ROOT, "include")


def _need(tool):
    path = shutil.which(tool)
    if path is None:
        pytest.skip(f"{tool} not found")
    return path


def test_c11_caller(tmp_path):
    if not os.path.exists(mxq.LIB_PATH):
        pytest.fail("libmxq.so is missing: build the library")
    gcc = _need("gcc")
    exe = str(tmp_path / "mxq_abi_check")
    libdir = os.path.dirname(mxq.LIB_PATH)
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", INC,
                    os.path.join(SRC, "mxq_abi_check.c"), "-o", exe, "-L", libdir, "-lmxq",
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True, text=True)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    r = subprocess.run([exe], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "all checks passed" in r.stdout


def test_cxx_caller(tmp_path):
    gxx = _need("g++")
    subprocess.run([gxx, "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", INC, "-c",
                    os.path.join(SRC, "mxq_header_cxx.cpp"), "-o", str(tmp_path / "h.o")],
                   check=True, capture_output=True, text=True)
