"""Builds libsdv.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree, and the
cross-check library libsdv_xcheck.so that the GPU tests load beside it.

Each source compiles to its own object under _build/ (in parallel).  The C-ABI source
compiles twice: as is for libsdv.so, and with SDV_XCHECK for libsdv_xcheck.so, whose
extra sdv_xcheck_* entry points take the kernel family as an argument so that the tests
can run every kernel implementation on the same inputs.  Both libraries link the same
kernel objects.
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
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsdv.so")
XCHECK_LIB = os.path.join(PKG, "libsdv_xcheck.so")
API_SOURCE = "sdv_api.cpp"
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    # packed fp32 instructions are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fno-gpu-flush-denormals-to-zero",
    f"-I{os.path.join(ROOT, 'include')}",
]


# Per-file additions.  The flat persistent kernel and the per-wave kernels hold their
# accumulators in ordinary VGPRs: at one workgroup per CU the compiler otherwise parks
# them in AGPRs and copies them back and forth around every block's products (per-wave
# kernel on 64-row dense pairs: 100 -> 94 us; its persistent form 109 -> 88 us, no
# longer spilling; the sparse and paged defaults unchanged within 1 us).
EXTRA = {
    "k_attn_flat.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "k_attn_waves.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def _compile(job, verbose: bool) -> str:
    src, defines, suffix = job
    obj = os.path.join(BUILD, os.path.basename(src) + suffix + ".o")
    cmd = [hipcc(), *COMMON, *defines, *EXTRA.get(os.path.basename(src), []), "-x", "hip", "-c",
           src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, lib)


def build_library(verbose: bool = False, jobs: int = 8) -> str:
    """Builds both libraries; returns the product library's path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs_list = [(s, [], "") for s in srcs]
    api = [s for s in srcs if os.path.basename(s) == API_SOURCE]
    jobs_list += [(s, ["-DSDV_XCHECK"], ".xcheck") for s in api]
    with cf.ThreadPoolExecutor(max_workers=min(jobs, len(jobs_list))) as ex:
        objs = list(ex.map(lambda j: _compile(j, verbose), jobs_list))
    plain = objs[:len(srcs)]
    xobj = objs[len(srcs):]
    kernels = [o for s, o in zip(srcs, plain) if os.path.basename(s) != API_SOURCE]
    _link(plain, LIB)
    _link(kernels + xobj, XCHECK_LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
