"""Build libmxq.so (the HIP kernels and the C ABI of include/mxq.h) for gfx950.

    python -m nvfp4_quantization_amd.build        # or: python nvfp4_quantization_amd/build.py

Compiled in-tree with hipcc; always rebuilds.  Flags:
  -ffp-contract=off   no FMA contraction: every a*b+c in the sources rounds twice
                      unless written as an explicit fma (the kernels are bit-exact)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed FP32 instructions (v_pk_add/mul/fma_f32)
  -mllvm -pragma-unroll-threshold=1000000
                      fully unroll every '#pragma unroll' loop, however large: a
                      kept loop would index register arrays dynamically and move
                      them to scratch memory
FP32 denormals are kept and FP32 division is correctly rounded (hipcc defaults).
The single-read kernels (mxq_nvfp4_fused_*.hip) are also built with
  -mllvm -disable-machine-licm
                      their per-item loop would otherwise keep loop-invariant lane
                      addresses live through the quantizing passes, whose registers
                      are at the limit, and spill a third of the tile
_build/libmxq_ceiling.so holds the benchmark's streaming read and copy kernels (the
measured HBM ceilings; not part of the quantization ABI).
_build/libmxq_selftest.so holds test-only kernels (tests/hip/mxq_selftest.hip) that
sweep the hardware conversions over their whole input range; nothing in the package
loads it.
A further library, _build/libmxq_defer0.so, is the same code with the single-read
kernels built with MXQ_FUSED_DEFER_TICKS=0: every waiting item gives up at once and
leaves its tiles to its section's last item, which the deferral test checks against
the oracle (the condition only a device short of room produces otherwise).
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "_build")
LIB = os.path.join(OUT, "libmxq.so")
LIB_DEFER0 = os.path.join(OUT, "libmxq_defer0.so")
LIB_CEILING = os.path.join(OUT, "libmxq_ceiling.so")     # the benchmark's HBM read / copy ceilings
LIB_SELFTEST = os.path.join(OUT, "libmxq_selftest.so")   # the tests' conversion sweeps
SELFTEST_SRC = os.path.join(ROOT, "tests", "hip", "mxq_selftest.hip")
ARCH = "gfx950"

HIP_SOURCES = ["mxq_fp8.hip", "mxq_fp8_block.hip", "mxq_swiglu_fp8.hip", "mxq_dsa_nvfp4.hip", "mxq_nvfp4.hip", "mxq_nvfp4_quant_rne.hip", "mxq_nvfp4_quant_sr.hip",
               "mxq_nvfp4_quant_rne_aout.hip", "mxq_nvfp4_quant_sr_aout.hip",
               "mxq_nvfp4_fused_rne.hip", "mxq_nvfp4_fused_sr.hip", "mxq_noalloc.hip"]
HOST_SOURCES = ["mxq_api.cpp"]
FUSED_SOURCES = ("mxq_nvfp4_fused_rne.hip", "mxq_nvfp4_fused_sr.hip")
EXTRA = {src: ["-mllvm", "-disable-machine-licm"] for src in FUSED_SOURCES}
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall", "-Werror", "-I", "/opt/rocm/include",
          "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics", "-mllvm", "-pragma-unroll-threshold=1000000"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the mxq HIP library cannot be built")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; drop that line
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(OUT, exist_ok=True)
    cc = hipcc()
    jobs = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        cmd = [cc, *COMMON, *DEVICE, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps:
            cmd += ["-save-temps=obj"]
        jobs.append(cmd)
        objs.append(obj)
    for src in HOST_SOURCES:
        obj = os.path.join(OUT, src + ".o")
        jobs.append([cc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the deferral test build: the single-read units again, waits of zero ticks
    defer_objs = []
    for src in FUSED_SOURCES:
        obj = os.path.join(OUT, src + ".defer0.o")
        jobs.append([cc, *COMMON, *DEVICE, *EXTRA.get(src, []), "-DMXQ_FUSED_DEFER_TICKS=0", "-c",
                     os.path.join(CSRC, src), "-o", obj])
        defer_objs.append(obj)
    ceiling_obj = os.path.join(OUT, "mxq_ceiling.hip.o")
    jobs.append([cc, *COMMON, *DEVICE, "-c", os.path.join(CSRC, "mxq_ceiling.hip"), "-o", ceiling_obj])
    selftest_obj = os.path.join(OUT, "mxq_selftest.hip.o")
    jobs.append([cc, *COMMON, *DEVICE, "-c", SELFTEST_SRC, "-o", selftest_obj])
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        list(ex.map(lambda c: _run(c, verbose), jobs))
    tmp = LIB_CEILING + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, ceiling_obj], verbose)
    os.replace(tmp, LIB_CEILING)
    tmp = LIB_SELFTEST + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, selftest_obj], verbose)
    os.replace(tmp, LIB_SELFTEST)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    fused_objs = {os.path.join(OUT, src + ".o") for src in FUSED_SOURCES}
    tmp = LIB_DEFER0 + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp,
          *[o for o in objs if o not in fused_objs], *defer_objs], verbose)
    os.replace(tmp, LIB_DEFER0)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, save_temps="--save-temps" in sys.argv))
