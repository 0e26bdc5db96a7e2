"""Build the CPU oracle (test infrastructure) into oracle/_build/libmxq_oracle.so.

Plain gcc, no vector extensions, no fast-math and no FMA contraction, so every
float operation in mxq_oracle.c is one correctly rounded IEEE binary32 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(OUT_DIR, "libmxq_oracle.so")
CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build(verbose: bool = False) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    src = os.path.join(HERE, "mxq_oracle.c")
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
