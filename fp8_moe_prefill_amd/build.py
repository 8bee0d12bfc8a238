"""Build the HIP library ``libfp8moe.so`` in-tree for gfx950 with hipcc.

Usage: ``python fp8_moe_prefill_amd/build.py`` (or ``build()`` of ``__graft_entry__``). Every
call recompiles; objects go to ``fp8_moe_prefill_amd/_build/`` and the library next to this
file. It imports nothing from the package, so it runs while the library is stale or absent.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfp8moe.so")

KERNELS = ["quant_act.hip", "route_permute.hip", "bank_pack.hip", "grouped_gemm.hip",
           "dense_gemm.hip", "combine.hip", "rmsnorm.hip", "bf16_gemm.hip",
           "attention.hip"]
HOST = ["capi.cpp"]

ARCH = "gfx950"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = [f"--offload-arch={ARCH}", "-fno-gpu-rdc",
          # packed fp32 VALU ops off (see the library's numerics notes)
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
          # MFMA in its VGPR form (C/D in VGPRs), so the VALU fold reads the MFMA result
          # without accumulator-register copies
          "-mllvm", "-amdgpu-mfma-vgpr-form"]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    jobs = []
    for src in KERNELS:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([hipcc, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE)
    for src in HOST:
        obj = os.path.join(BUILD, src.replace(".cpp", ".o"))
        jobs.append([hipcc, "-c", os.path.join(CSRC, src), "-o", obj] + COMMON)
    with ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        for r in ex.map(_run, jobs):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout, r.stderr, file=sys.stderr)
    objs = [os.path.join(BUILD, s.rsplit(".", 1)[0] + ".o") for s in KERNELS + HOST]
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
