"""Build the CPU oracle (plain C, fp64) into oracle/liboracle.so with gcc.

Test infrastructure only: the library it builds is loaded by the test suite,
the smoke check and the benchmark's CPU-baseline leg, never by the GPU path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gqa_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle; always recompiles.  Returns the library path."""
    tmp = LIB + ".tmp"
    cmd = [
        "gcc", "-std=c11", "-D_GNU_SOURCE", "-O2", "-fPIC", "-shared",
        # IEEE fp64 exactly as written: no contraction into FMA, no fast-math.
        "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra",
        "-o", tmp, SRC, "-lm", "-lpthread",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
