"""Build libnvfp4.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc.

Run ``python -m skinny_gemm_nvfp4_amd.build`` (or ``__graft_entry__.build()``). The library lands
next to this file; the Python binding loads it from there and refuses to run without it.

Flags that matter for results:
  -Xclang -target-feature -Xclang -packed-fp32-ops
        no packed fp32 arithmetic anywhere in the device code.
  -ffp-contract=off
        no fused multiply-add where the source writes a multiply and an add: the quantisation
        recipe rounds every fp32 step on its own.
  -fhip-fp32-correctly-rounded-divide-sqrt
        fp32 division is correctly rounded (the recipe divides twice).
  -mllvm -amdgpu-mfma-vgpr-form
        matrix-core accumulators in ordinary VGPRs: without it the compiler moves the 16x16
        accumulators through AGPRs with copies around every MFMA of the unrolled tile loops.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libnvfp4.so")
SOURCES = ["api.cpp", "pack.hip", "gemm.hip", "grouped.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the NVFP4 HIP library cannot be built")


def compile_flags() -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fno-gpu-rdc",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
            "-mllvm", "-amdgpu-mfma-vgpr-form",
            "-Wall", "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]


def _compile(src: str, verbose: bool, flags: list, out_dir: str) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *flags, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is harmless.
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    return obj


def _build(out: str, flags: list, link_flags: list, obj_dir: str, verbose: bool) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, flags, obj_dir), SOURCES))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *link_flags, "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link of {os.path.basename(out)} failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile every source and link libnvfp4.so. Always recompiles."""
    return _build(LIB, compile_flags(), [], BUILD_DIR, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
