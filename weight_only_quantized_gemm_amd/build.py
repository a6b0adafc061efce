"""Build libwq.so (the HIP kernels and the C ABI) in-tree for gfx950 with hipcc."""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libwq.so")
SOURCES = ["wq_api.hip", "wq_repack.hip", "wq_gemm_small.hip", "wq_gemm_tile.hip",
           "wq_measure.hip"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libwq.so")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 into weight_only_quantized_gemm_amd/libwq.so."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
           # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # keep MFMA accumulators in arch VGPRs: the kernels update them with VALU ops
           "-mllvm", "-amdgpu-mfma-vgpr-form=1",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-o", tmp] + [os.path.join(CSRC, s) for s in SOURCES] + (extra or [])
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if verbose and res.stderr:
        sys.stderr.write("\n".join(l for l in res.stderr.splitlines()
                                   if "packed-fp32-ops" not in l) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
