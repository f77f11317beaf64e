"""Build the gfx950 shared library ``libfp_prefill.so`` in the package directory.

Translation units:
  plan_kernels.hip   selection kernels, compiled with -ffp-contract=off (the
                     canonical arithmetic forbids implicit fused multiply-adds)
  attn_kernels.hip   attention kernels
  fp_api.cpp         host C ABI
All device code is compiled with packed-fp32 instructions disabled.

Usage: python -m sparse_long_context_last_amd.build [-v]
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp_prefill.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-I", CSRC, "-I", INCLUDE,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-flush-denormals-to-zero",
          "-Wall", "-Wno-unused-command-line-argument"]

UNITS = {
    "plan_kernels.hip": ["-ffp-contract=off", "-fno-fast-math"],
    "attn_kernels.hip": [],
    "fp_api.cpp": ["-x", "hip"],
}


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose: bool = False) -> str:
    """Compile every translation unit for gfx950 and link libfp_prefill.so."""
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    objs = []
    for src, flags in UNITS.items():
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        jobs.append([cc, *COMMON, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with cf.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for f in [ex.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
