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


HOST_CHECK_LIB = os.path.join(HERE, "libgated_attn_hostcheck.so")
CLANGXX = os.environ.get("GA_CLANGXX", "/opt/rocm/llvm/bin/clang++")


def build_host_check(sanitize: bool = False, out: str = HOST_CHECK_LIB, verbose: bool = False) -> str:
    """The C ABI (capi.cpp) linked against csrc/host_stub.cpp instead of the
    HIP runtime and the kernels: every host-side path of the ABI -- argument
    checks, split plans, workspace layout, the device-arch decision, the
    no-allocation entry point's scratch lookup -- runs on a machine without a
    GPU and reports what it would have launched.  ``sanitize``: AddressSanitizer
    and UndefinedBehaviorSanitizer on the host code (load with the clang ASan
    runtime preloaded)."""
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"] if sanitize else []
    build_dir = os.path.join(HERE, "_build")
    os.makedirs(build_dir, exist_ok=True)
    tag = "_san" if sanitize else ""
    objs = []
    for src, host_only in (("capi.cpp", False), ("host_stub.cpp", True)):
        obj = os.path.join(build_dir, f"hostcheck_{src}{tag}.o")
        cmd = [HIPCC, "-x", "hip", *COMMON_FLAGS, "-g", *san,
               *(["--cuda-host-only"] if host_only else []),
               "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}{r.stderr}")
        objs.append(obj)
    # linked with clang++, not hipcc, so no HIP runtime is pulled in; symbols
    # bind inside the library first, so the stubs answer capi.cpp's calls even
    # in a process where torch has loaded the real runtime
    tmp = out + ".tmp"
    link_san = ["-fsanitize=address,undefined", "-shared-libasan"] if sanitize else []
    cmd = [CLANGXX, "-shared", "-fPIC", "-Wl,-Bsymbolic", "-Wl,--no-undefined", *link_san,
           "-o", tmp, *objs, "-lpthread"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--host-check" in sys.argv:
        print(build_host_check(sanitize="--sanitize" in sys.argv, verbose="-v" in sys.argv))
