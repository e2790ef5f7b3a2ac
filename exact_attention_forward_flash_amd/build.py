"""Builds libwf.so (the HIP kernels and the C ABI of include/wf.h) in-tree for gfx950.

    python -m exact_attention_forward_flash_amd.build

Every translation unit under csrc/ is compiled with hipcc in parallel into _build/, then
linked into exact_attention_forward_flash_amd/libwf.so (replaced atomically).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libwf.so")
ARCH = os.environ.get("WF_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # packed fp32 VALU forms are kept out of the generated code on purpose
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


# 64-query-wave kernels: MFMAs the compiler generates keep VGPR accumulators (their O^T
# accumulators are placed in AGPRs explicitly).
W64_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def flags_for(src):
    return FLAGS + (W64_FLAGS if src.endswith("_w64.hip") else [])


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags_for(src), "-c", src, "-o", obj]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, time.time() - t0


def build(verbose=True, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 4)))
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        slow = ", ".join(f"{os.path.basename(o)[:-2]} {t:.0f}s" for o, t in results)
        print(f"built {LIB} in {time.time() - t0:.1f}s ({slow})", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
