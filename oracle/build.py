"""Compile the CPU oracle (plain C, gcc, no HIP) into oracle/libbeam_oracle.so.

The oracle is test infrastructure: the tests, the smoke check and the
benchmark's CPU-baseline leg load it; the GPU library never does.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "beam_oracle.c")
LIB = os.path.join(HERE, "libbeam_oracle.so")


# -ffp-contract=off: no a*b+c fusion beyond the fma() calls the routing
# specification writes out; no -ffast-math, so sums keep their order.
FLAGS = ["-O2", "-std=gnu11", "-fPIC", "-shared", "-fopenmp",
         "-ffp-contract=off", "-fno-fast-math", "-Wall"]


def compile_to(src: str, out: str, extra=(), verbose: bool = False) -> str:
    """Compile one C source file into the shared library `out`."""
    cmd = ["gcc", *FLAGS, *extra, "-o", out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False) -> str:
    return compile_to(SRC, LIB, verbose=verbose)


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
