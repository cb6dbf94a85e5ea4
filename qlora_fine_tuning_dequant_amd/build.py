"""Builds libqlx.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every translation unit compiles in parallel to an object file under
``_build/``; the objects link into ``libqlx.so`` next to this file."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libqlx.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["k_nf4.hip", "k_gemm.hip", "k_elem.hip", "attention.hip", "optim.hip", "merge.hip", "layer.hip", "api.hip",
           "source.hip", "prof.hip", "peaks.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
         # packed fp32 instructions stay off (see the build notes)
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function",
         "-Wno-unused-command-line-argument",
         # MFMA accumulators in ordinary VGPRs: with AGPR accumulators the
         # register allocator splits them between the two files and shuffles
         # them through v_accvgpr moves in every loop iteration (measured: a
         # 16x16x32 bf16 MFMA loop at 56% of peak with the moves, 95% without)
         "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
EXTRA: dict = {}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32" not in l)
    if warn:
        print(f"[build] {src}: {warn}", file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"[build] {OUT}")
    return OUT


if __name__ == "__main__":
    build()
