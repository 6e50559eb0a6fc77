"""Compile the HIP sources of the MoE layer into libexpert_layer_amd.so (gfx950).

    python -m expert_layer_amd.build

Every source is compiled with hipcc for --offload-arch=gfx950 (packed fp32
instructions disabled) into _build/, then linked into the package directory,
where the binding loads it.  It always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libexpert_layer_amd.so")
SOURCES = ["capi.cpp", "route.hip", "permute.hip", "gemm_bf16.hip", "gemm_fp8.hip", "gemm_e4m3.hip", "gemm_f32.hip", "combine.hip"]
VGPR_FORM = {"gemm_fp8.hip", "gemm_e4m3.hip"}
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if c and os.path.exists(c):
            return c
    return "hipcc"


def _flags(src: str):
    f = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", f"-I{os.path.join(ROOT, 'include')}"]
    if src.endswith(".hip"):
        f += [f"--offload-arch={ARCH}", "-x", "hip",
              "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
              "-munsafe-fp-atomics"]
        if src in VGPR_FORM:
            # MFMA results in VGPRs: the fp8 path promotes every MFMA result on the VALU
            f += ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]
    else:
        f += ["-D__HIP_PLATFORM_AMD__"]
    return f


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + _flags(src) + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
