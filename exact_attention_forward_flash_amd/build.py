"""Builds libwf.so (the HIP kernels and the C ABI of include/wf.h) in-tree for gfx950.

    python -m exact_attention_forward_flash_amd.build [--sanitize]

Every translation unit under csrc/ is compiled with hipcc in parallel into _build/, then
linked into exact_attention_forward_flash_amd/libwf.so (replaced atomically).
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
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


def source_hash():
    """sha256 over the target, the compile flags and every source and header the library is
    built from; stored in the library (wf_build_id) and checked when the package loads it."""
    h = hashlib.sha256()
    h.update(" ".join([ARCH, *FLAGS[1:], *W64_FLAGS]).replace(ROOT, "").encode())
    files = [os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp", ".hpp", ".h"))]
    inc = os.path.join(ROOT, "include")
    files += [os.path.join(inc, f) for f in os.listdir(inc) if f.endswith(".h")]
    for path in sorted(files, key=lambda p: os.path.relpath(p, ROOT)):
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def _build_id_source():
    os.makedirs(BUILD, exist_ok=True)
    path = os.path.join(BUILD, "wf_build_id.cpp")
    text = ('extern "C" const char* wf_build_id(void) { return "%s"; }\n' % source_hash())
    old = open(path).read() if os.path.exists(path) else None
    if old != text:
        with open(path, "w") as f:
            f.write(text)
    return path


# 64-query-wave kernels: MFMAs the compiler generates keep VGPR accumulators (their O^T
# accumulators are placed in AGPRs explicitly).
W64_FLAGS = ["-mllvm", "-amdgpu-mfma-vgpr-form"]


def flags_for(src):
    return FLAGS + (W64_FLAGS if src.endswith("_w64.hip") else [])


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for the host code of every unit;
# the device code is built exactly as in the normal library.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
SAN_BUILD = os.path.join(BUILD, "san")
SAN_LIB = os.path.join(SAN_BUILD, "libwf_san.so")


def sanitizer_runtime():
    """The clang AddressSanitizer runtime (with UBSan) a process must preload to load SAN_LIB."""
    rd = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin",
                         "clang"), "-print-resource-dir"], capture_output=True, text=True).stdout.strip()
    path = os.path.join(rd, "lib", "linux", "libclang_rt.asan-x86_64.so")
    if not os.path.exists(path):
        raise RuntimeError(f"no AddressSanitizer runtime at {path}")
    return path


def _compile(src, out_dir=None, extra=()):
    obj = os.path.join(out_dir or BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *flags_for(src), *extra, "-c", src, "-o", obj]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (p.stdout + p.stderr).splitlines() if noise not in l)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, time.time() - t0


def build(verbose=True, jobs=None, sanitize=False):
    """Builds libwf.so; with sanitize, builds SAN_LIB instead (same sources, host code under
    ASan + UBSan, loaded through WF_LIBRARY with sanitizer_runtime() preloaded)."""
    out_dir, lib = (SAN_BUILD, SAN_LIB) if sanitize else (BUILD, LIB)
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources() + [_build_id_source()]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 4)))
    t0 = time.time()
    extra = SANITIZE_HOST if sanitize else ()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, out_dir, extra), srcs))
    objs = [o for o, _ in results]
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stdout}\n{p.stderr}")
    os.replace(tmp, lib)
    if verbose:
        slow = ", ".join(f"{os.path.basename(o)[:-2]} {t:.0f}s" for o, t in results)
        print(f"built {lib} in {time.time() - t0:.1f}s ({slow})", flush=True)
    return lib


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
