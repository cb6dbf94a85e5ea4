"""Builds libqlx.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

Every translation unit compiles in parallel to an object file under
``_build/``; the objects link into ``libqlx.so`` next to this file.

``build(sanitize="address" | "thread")`` builds the host side of the library
instrumented with AddressSanitizer or ThreadSanitizer instead (host code only:
``-Xarch_host -fsanitize=...``; the device code is the ordinary one), into
``_build/<asan|tsan>/libqlx.so``, for the CPU tests of the host logic (the
disk reader threads and their bounce buffers, argument validation). Such a
library is only ever loaded by those tests, through ``QLX_LIB`` with the
sanitizer runtime preloaded (``sanitizer_env``)."""
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


# host-sanitizer builds: the instrumentation applies to host code only
SAN = {"address": ("asan", ["-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address"]),
       # (gcc's older TSan runtime has no __tsan_memcpy: memory intrinsics stay plain calls)
       "thread": ("tsan", ["-O1", "-g", "-Xarch_host", "-fsanitize=thread", "-mllvm",
                           "-tsan-instrument-memintrinsics=false"])}
# runtimes to preload into an uninstrumented python (clang's ASan; gcc's TSan
# runtime serves clang's instrumentation, the ROCm toolchain ships no TSan one)
SAN_RUNTIME = {"address": "/opt/rocm/lib/llvm/lib/clang/{ver}/lib/linux/libclang_rt.asan-x86_64.so",
               "thread": "/usr/lib/x86_64-linux-gnu/libtsan.so.0"}


def _compile(src: str, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, src.replace(".hip", ".o"))
    cmd = [HIPCC, *FLAGS, *EXTRA.get(src, []), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "warning" in l and "packed-fp32" not in l)
    if warn:
        print(f"[build] {src}: {warn}", file=sys.stderr)
    return obj


def build(verbose: bool = True, sanitize: str | None = None) -> str:
    build_dir, out, extra, link = BUILD, OUT, [], []
    if sanitize is not None:
        sub, extra = SAN[sanitize]
        build_dir = os.path.join(BUILD, sub)
        out = os.path.join(build_dir, "libqlx.so")
        link = ["-Xarch_host", f"-fsanitize={sanitize}"]
    os.makedirs(build_dir, exist_ok=True)
    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"[build] {out}")
    return out


def sanitizer_env(sanitize: str, lib_path: str) -> dict:
    """Environment for a python process that loads the sanitized library."""
    import glob
    rt = SAN_RUNTIME[sanitize]
    if "{ver}" in rt:
        found = sorted(glob.glob(rt.replace("{ver}", "*")))
        if not found:
            raise FileNotFoundError(rt)
        rt = found[-1]
    env = dict(os.environ)
    env["QLX_LIB"] = lib_path
    env["LD_PRELOAD"] = rt
    # python itself is not instrumented: no leak report of its arenas, and the
    # runtime need not come first among the libraries it was started with
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:halt_on_error=1"
    env["TSAN_OPTIONS"] = "halt_on_error=1:report_signal_unsafe=0"
    return env


if __name__ == "__main__":
    build()
