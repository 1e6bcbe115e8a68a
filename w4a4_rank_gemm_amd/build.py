"""Build libtwq.so for gfx950 with hipcc (in-tree: w4a4_rank_gemm_amd/lib/libtwq.so)."""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "lib", "libtwq.so")
SOURCES = ["act_quant.hip", "pack_weight.hip", "dual_linear.hip", "lowrank_int4.hip", "noalloc.hip", "fold.hip", "plan.cpp", "twq_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libtwq)")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # eq. (1) divides in binary32; the quantizer relies on the correctly rounded form
        "-fhip-fp32-correctly-rounded-divide-sqrt",
        # no packed fp32 arithmetic anywhere in the device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    ]


def _stale(src: str, out: str) -> bool:
    """True if out is missing or older than its source or any header it may include."""
    if not os.path.exists(out):
        return True
    deps = [os.path.join(CSRC, src)] + [os.path.join(CSRC, h) for h in os.listdir(CSRC) if h.endswith(".h")]
    deps.append(os.path.join(ROOT, "include", "twq.h"))
    t = os.path.getmtime(out)
    return any(os.path.getmtime(d) > t for d in deps)


def _compile(src: str, incremental: bool = False) -> str:
    out = os.path.join(OBJ, os.path.basename(src) + ".o")
    if incremental and not _stale(src, out):
        return out
    cmd = [hipcc(), *compile_flags(), "-c", os.path.join(CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return out


def build(verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (incremental: only those older than their inputs) and link."""
    os.makedirs(OBJ, exist_ok=True)
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, incremental), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    import sys
    build(verbose=True, incremental="--incremental" in sys.argv)
