"""Build step: compile the HIP kernels and the C ABI into ``libfa.so`` inside this package.

Every source is compiled for gfx950 only, with packed-fp32 instruction selection switched off, then
linked into one shared library.  Objects go to ``_build/`` at the repository root.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_host.cpp", "fa_fwd.hip", "fa_fwd_f32.hip", "fa_fwd_fp8.hip", "fa_fp8_prep.hip", "fa_bwd.hip", "fa_decode.hip", "fa_naive.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libfa.so)")


def _flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
        "-Wall", "-Wno-unused-function",
    ]


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every source and link ``libfa.so``; returns the library path.  Always rebuilds."""
    cc = hipcc()
    out_dir = os.path.join(ROOT, "_build")
    os.makedirs(out_dir, exist_ok=True)

    def compile_one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [cc, *_flags(), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        noise = "is not a recognized feature for this target"
        err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{err}")
        if verbose and err.strip():
            print(err, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
