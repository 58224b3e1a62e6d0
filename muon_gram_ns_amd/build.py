"""Build libgns.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python muon_gram_ns_amd/build.py        # or __graft_entry__.build()

(run it by path: importing the package loads the library it is about to rebuild)

Every source is compiled for gfx950 only.  Packed-fp32 instructions are disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); the Dion3 and Muon files are compiled
with -ffp-contract=off so their fp32 update arithmetic is not fused into multiply-adds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libgns.so")

SOURCES = {
    "gemm_symm.hip": [],
    "gemm_rect.hip": [],
    "elementwise.hip": [],
    "dion3.hip": ["-ffp-contract=off"],
    "muon.hip": ["-ffp-contract=off"],
    "gns_abi.cpp": [],
}

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def _compile(src: str, extra: list[str], verbose: bool) -> str:
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + extra
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def hip_runtime_for_link() -> str:
    return "/opt/rocm/lib/libamdhip64.so"


def clangxx() -> str:
    for c in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("clang++ not found")


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(5, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(kv[0], kv[1], verbose), SOURCES.items()))
    tmp = LIB + ".tmp"
    # host link only (each object already embeds its gfx950 code object); plain
    # clang++ so that no other HIP runtime is added to the dependencies
    cmd = [clangxx(), "-shared", "-fPIC", "-o", tmp] + objs + [hip_runtime_for_link(), "-Wl,--no-undefined",
                                                                  "-lstdc++", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
