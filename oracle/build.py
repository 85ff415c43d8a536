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


def build(verbose: bool = False, sanitize: bool = False, out: str = LIB) -> str:
    """Compile the oracle; always recompiles.  Returns the library path.
    ``sanitize``: clang with AddressSanitizer and UndefinedBehaviorSanitizer
    (load with the clang ASan runtime preloaded)."""
    tmp = out + ".tmp"
    cc = ["gcc", "-O2"]
    if sanitize:
        cc = ["/opt/rocm/llvm/bin/clang", "-O1", "-g", "-fno-omit-frame-pointer",
              "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libasan"]
    cmd = [
        *cc, "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
        # IEEE fp64 exactly as written: no contraction into FMA, no fast-math.
        "-ffp-contract=off", "-fno-fast-math",
        "-Wall", "-Wextra",
        "-o", tmp, SRC, "-lm", "-lpthread",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, sanitize="--sanitize" in sys.argv))
