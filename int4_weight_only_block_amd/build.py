"""Build libq4dec.so (HIP, gfx950 only) in-tree with hipcc.

Every .hip file under csrc/ is compiled to an object and the objects are linked
into one shared library next to this file. Called by __graft_entry__.build()
and usable as ``python -m int4_weight_only_block_amd.build``.

``build(asan=True)`` builds libq4dec_asan.so: the same sources with the host
code (argument checks, plans, launch set-up) instrumented by AddressSanitizer;
device code is compiled as usual. It is for CPU runs of the host paths, with
the sanitizer runtime preloaded (see ``asan_runtime()``).

``build(debug=True)`` (or ``Q4DEC_DEBUG=1 python -m
int4_weight_only_block_amd.build``) builds libq4dec_debug.so with
-DQ4DEC_DEBUG=1: every kernel checks its launch contract on the device and
records failures for q4dec_debug_status().
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "libq4dec.so")
ASAN_LIB_PATH = os.path.join(HERE, "libq4dec_asan.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libq4dec_debug.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # keep packed fp32 VALU ops out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


# host-only AddressSanitizer (each flag bound to the host pass)
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ASAN_LINK_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-shared-libsan"]


# per-file additions: the S=64 GEMM folds every MFMA result on the VALU, so
# its MFMAs write VGPRs directly instead of going through AGPR copies
FILE_FLAGS = {
    "q4_gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP toolchain is required to build libq4dec")
    return path


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that libq4dec_asan.so links
    against (to be preloaded into an uninstrumented python)."""
    res = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "lib", "llvm", "bin",
                                       "clang"), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode == 0 and os.path.isabs(path) and os.path.exists(path):
        return path
    found = sorted(glob.glob("/opt/rocm*/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return found[-1]


def _compile(src: str, verbose: bool, build_dir: str, extra: list) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    return obj


def build(verbose: bool = False, jobs: int | None = None, asan: bool = False, debug: bool = False) -> str:
    if asan and debug:
        raise ValueError("build one variant at a time")
    build_dir = os.path.join(BUILD_DIR, "asan" if asan else "debug") if (asan or debug) else BUILD_DIR
    lib_path = ASAN_LIB_PATH if asan else DEBUG_LIB_PATH if debug else LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if not sources:
        raise RuntimeError("no HIP sources found")
    jobs = jobs or min(len(sources), max(1, (os.cpu_count() or 4)))
    extra = ASAN_FLAGS if asan else ["-DQ4DEC_DEBUG=1"] if debug else []
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, build_dir, extra), sources))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *(ASAN_LINK_FLAGS if asan else []), "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, asan="--asan" in sys.argv,
                debug="--debug" in sys.argv or os.environ.get("Q4DEC_DEBUG", "0") not in ("", "0")))
