"""Build libm3.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m selective_state_space_mamba3_amd.build [-j N] [--verbose]

Objects go to <repo>/_build/; the shared library is written next to this
file so that it ships with the source tree.
"""

from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(REPO, "_build")
LIB_NAME = "libm3.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)

SOURCES = ["abi.cpp", "scan_fwd.hip", "siso_step.hip", "mimo_step.hip", "preprocess.hip", "scan_bwd.hip",
           "preprocess_bwd.hip"]

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 arithmetic on the device
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-I", os.path.join(REPO, "include"), "-c",
           os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = (res.stdout + res.stderr).strip()
    # the host pass does not know the device-only target feature; that note is harmless
    lines = [ln for ln in out.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if lines and verbose:
        print("\n".join(lines), flush=True)
    return obj


def build(jobs: int = 4, verbose: bool = False) -> str:
    """Compile every source and link libm3.so; return the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


ASAN_DIR = os.path.join(BUILD_DIR, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libm3_asan.so")


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that hipcc's host pass links against."""
    clang = os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin", "clang")
    if not os.path.exists(clang):
        clang = shutil.which("clang") or clang
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError(f"AddressSanitizer runtime not found (clang printed {path!r})")
    return path


def build_asan(verbose: bool = False) -> str:
    """Host-side AddressSanitizer build of the C ABI layer, for CPU tests.

    abi.cpp (argument validation, plans, error text, the scratch set-up) is
    compiled with -fsanitize=address on the host pass only (the device code
    is unchanged) and linked with the kernels' regular objects into
    _build/asan/libm3_asan.so.  The library carries no sanitizer runtime: a
    process loads it with asan_runtime() preloaded."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    others = []
    for src in SOURCES:
        if src == "abi.cpp":
            continue
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        others.append(obj if os.path.exists(obj) else _compile(src, verbose))
    obj = os.path.join(ASAN_DIR, "abi.o")
    cmd = [hipcc(), "-x", "hip", *COMMON_FLAGS, "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fno-omit-frame-pointer", "-I", os.path.join(REPO, "include"), "-c", os.path.join(CSRC, "abi.cpp"),
           "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc (asan) failed for abi.cpp:\n{res.stdout}{res.stderr}")
    tmp = ASAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", obj, *others,
           "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"asan link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("-j", "--jobs", type=int, default=min(8, os.cpu_count() or 4))
    ap.add_argument("--verbose", action="store_true")
    args = ap.parse_args(argv)
    path = build(args.jobs, args.verbose)
    print(path)
    return 0


if __name__ == "__main__":
    sys.exit(main())
