"""Build libdspark_attn.so in-tree with hipcc for gfx950.

    python speculative_decoding_draft_amd/build.py

(run as a file, not with -m: importing the package loads the library.)

Compiles every source under csrc/ (in parallel) and links the shared library
next to this file.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdspark_attn.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # the code object is loaded by the HIP runtime torch ships, which may be
    # older than this compiler: keep the bundle uncompressed
    "--no-offload-compress",
    "-Wno-unused-function",
    # packed fp32 ops are disabled on purpose: hand-independent code paths
    # must not rely on v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
SOURCES = ["prep.hip", "generic.hip", "absorb.hip", "attn.hip", "uv.hip", "api.hip",
           "sampler.cpp", "bwd_misc.hip", "bwd_gemm.hip", "bwd_attn.hip", "layer.hip",
           "blas.hip", "loss.hip", "decode.hip", "fused.hip"]


def _hipcc() -> str:
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libdspark_attn.so")


def _compile(src: str, hipcc: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc, *COMMON_FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)
    return obj


def _hip_runtime_dir() -> str:
    """Directory of the HIP runtime that torch loads.  The library must use
    that same runtime: a second libamdhip64 in the process does not see the
    device, and torch's streams and allocations belong to torch's runtime."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is not None and spec.origin:
        d = os.path.join(os.path.dirname(spec.origin), "lib")
        if os.path.exists(os.path.join(d, "libamdhip64.so")):
            return d
    return "/opt/rocm/lib"


def build(verbose: bool = True, extra_flags=()) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(lambda s: _compile(s, hipcc, list(extra_flags)), SOURCES))
    tmp = LIB + ".tmp"
    rt = _hip_runtime_dir()
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc)), "..", "lib", "llvm", "bin",
                         "clang++")
    if not os.path.exists(clang):
        clang = "/opt/rocm/lib/llvm/bin/clang++"
    # rocBLAS (the MLA block's projections) from the same directory as the
    # HIP runtime, so that both are the instances torch has loaded
    cmd = [clang, "-shared", "-fPIC", "-o", tmp, *objs, f"-L{rt}", f"-Wl,-rpath,{rt}",
           "-l:libamdhip64.so", "-l:librocblas.so", "-Wl,--no-undefined", "-lstdc++", "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(extra_flags=sys.argv[1:])
