"""Build libqsa.so: the gfx950 kernels and the C ABI of include/qsa.h.

Ahead-of-time code objects for gfx950 only (no JIT).  Flags that matter for the numerics:
-ffp-contract=off (no FMA contraction: each product is rounded before it is added), no
fast-math, default IEEE denormal handling, and packed FP32 instructions disabled.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libqsa.so")
ARCH = "gfx950"
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

COMMON = ["-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", "-ffp-contract=off",
          "-fno-fast-math", "-Wall", "-I", INCLUDE, "-I", CSRC]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "is not a recognized feature for this target"
    out = "\n".join(l for l in r.stdout.splitlines() if noise not in l)
    if out.strip():
        print(out, file=sys.stderr)
    if r.returncode != 0:
        raise RuntimeError(f"build failed ({r.returncode}): {' '.join(cmd)}")


def build(hipcc="hipcc"):
    """Compile and link libqsa.so (always recompiles): every .hip kernel source of csrc/ and
    the C ABI layer."""
    import glob
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    for src in sorted(glob.glob(os.path.join(CSRC, "*.hip"))):
        obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
        _run([hipcc, *COMMON, *DEVICE, "-c", src, "-o", obj])
        objs.append(obj)
    aobj = os.path.join(BUILD, "qsa_api.o")
    _run([hipcc, *COMMON, "-x", "c++", "-D__HIP_PLATFORM_AMD__", "-I",
          os.path.join(ROCM, "include"), "-c", os.path.join(CSRC, "qsa_api.cpp"), "-o", aobj])
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", *objs, aobj, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
