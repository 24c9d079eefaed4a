"""Build the CPU oracle library (test infrastructure only; see qsa_ref.c's header).

gcc, C11, -O2 with IEEE semantics kept: no FMA contraction, no fast-math, SSE binary32
arithmetic (the x86-64 default), OpenMP for the row/block loops.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qsa_ref.c")
LIB = os.path.join(HERE, "libqsa_ref.so")

FLAGS = ["-std=c11", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
         "-fno-fast-math", "-mfpmath=sse", "-msse2", "-Wall", "-Wextra", "-Werror"]


def build(extra_flags=(), out=LIB):
    """Compile qsa_ref.c into `out` (always recompiles)."""
    cmd = ["gcc", *FLAGS, *extra_flags, SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build())
