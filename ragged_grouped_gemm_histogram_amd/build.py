"""Build libmoe_grouped.so in-tree with hipcc for gfx950.

Usage: ``python -m ragged_grouped_gemm_histogram_amd.build`` (or ``build()``).
Each HIP source is compiled to an object under ``_build/`` in parallel, then
linked into ``libmoe_grouped.so`` next to this file. No GPU is needed.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_NAME = "libmoe_grouped.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = ["abi.hip", "permute.hip", "gemm.hip", "unpermute.hip"]
ARCH = "gfx950"

# Packed-fp32 instructions stay off: every float operation is issued unpacked.
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in res.stdout.splitlines() if "packed-fp32-ops" not in line
                    and "warnings generated when compiling for host" not in line)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)
    return out


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every HIP source for gfx950 and link the shared library; returns its path."""
    cc = hipcc()
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs or min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


# Host-sanitizer build (CPU tests only): host code with AddressSanitizer and
# UndefinedBehaviorSanitizer. Each sanitizer flag is scoped to the host compilation
# with -Xarch_host; the device code is built as usual and never run from this library.
SAN_DIR = os.path.join(BUILD_DIR, "host_sanitized")
SAN_LIB_PATH = os.path.join(SAN_DIR, "libmoe_grouped_host_sanitized.so")
SAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def clangxx() -> str:
    path = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang++")
    return os.path.realpath(path) if os.path.exists(path) else "/opt/rocm/llvm/bin/clang++"


def sanitizer_runtime() -> str:
    """The shared AddressSanitizer runtime the sanitized library needs preloaded (LD_PRELOAD)."""
    res = subprocess.run([clangxx(), "-print-file-name=libclang_rt.asan-x86_64.so"], stdout=subprocess.PIPE, text=True)
    return res.stdout.strip()


def build_host_sanitized(verbose: bool = False) -> str:
    """Host-only objects with ASan and UBSan, linked with the shared sanitizer runtime; returns the path."""
    cc = hipcc()
    os.makedirs(SAN_DIR, exist_ok=True)
    flags = [f for f in HIP_FLAGS if f != "-O3"] + ["-O1", *SAN_HOST_FLAGS]
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(SAN_DIR, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1, 8)) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    rocm_lib = os.path.realpath(os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "lib"))
    _run([clangxx(), "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libasan", "-o", SAN_LIB_PATH, *objs,
          f"-L{rocm_lib}", "-lamdhip64", f"-Wl,-rpath,{rocm_lib}"], verbose)
    return SAN_LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
