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
# every translation unit in csrc/ (the kernel headers are included by them)
SOURCES = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
OBJ_DIR = os.path.join(PKG, "_build")  # per-source objects (git-ignored)


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the ROCm toolchain is required to build libwq.so")


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source for gfx950 into weight_only_quantized_gemm_amd/libwq.so: one
    hipcc per source in parallel (the kernel instances dominate), then one link."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(OBJ_DIR, exist_ok=True)
    flags = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # keep the compiler from forming packed-fp32 VALU ops (v_pk_*_f32)
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # keep MFMA accumulators in arch VGPRs: the kernels update them with VALU ops
             "-mllvm", "-amdgpu-mfma-vgpr-form=1",
             "-I", os.path.join(ROOT, "include"), "-I", CSRC] + (extra or [])

    def compile_one(src: str):
        obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
        cmd = flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    workers = max(1, min(len(SOURCES), os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        results = list(pool.map(compile_one, SOURCES))
    failed = [(src, res) for src, (_, res) in zip(SOURCES, results) if res.returncode != 0]
    for src, res in failed:
        sys.stderr.write(f"--- {src}\n" + res.stdout + res.stderr)
    if failed:
        raise RuntimeError("hipcc failed for " + ", ".join(src for src, _ in failed))
    if verbose:
        for src, (_, res) in zip(SOURCES, results):
            lines = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l]
            if lines:
                sys.stderr.write("\n".join(lines) + "\n")
    tmp = LIB + ".tmp"
    link = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-Wl,--no-undefined", "-o", tmp] + \
        [obj for obj, _ in results]
    res = subprocess.run(link, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc link failed with status {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
