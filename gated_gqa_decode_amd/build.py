"""Build libgated_attn.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Always recompiles; the library lands next to this file so that it travels with
the source tree and is found by the binding without installation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libgated_attn.so")
SOURCES = ["capi.cpp", "decode.hip", "prefill.hip", "qk_norm_rope.hip", "stream_read.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # Packed fp32 arithmetic stays off: plain fp32 VALU instructions only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False, extra_flags=None, out: str = LIB) -> str:
    extra = list(extra_flags or [])
    objs = []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC, *lang, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        # hipcc's host pass does not know the packed-fp32 target feature and says so
        msgs = [ln for ln in (r.stdout + r.stderr).splitlines()
                if "packed-fp32-ops" not in ln and ln.strip()]
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
        if msgs and verbose:
            print("\n".join(msgs), flush=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True, capture_output=not verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
