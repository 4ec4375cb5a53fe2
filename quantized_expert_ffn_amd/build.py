"""Build libmoe.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m quantized_expert_ffn_amd.build

Compiles every csrc/*.hip to an object under _build/ with hipcc and links
them into quantized_expert_ffn_amd/lib/libmoe.so. Always recompiles.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmoe.so")

ARCH = "gfx950"
# Packed fp32 vector instructions are kept out of every kernel; matrix-core
# results go to ordinary VGPRs (the epilogues consume them with VALU ops,
# which would otherwise first copy them out of AGPRs).
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=1"]
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Wno-unused-variable"] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: libmoe needs ROCm's hipcc to build")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + CFLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    workers = min(len(sources), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers) as pool:
        objs = list(pool.map(_compile, sources))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}", file=sys.stderr)
    return LIB


# The host ABI check: the ABI layer's translation unit with AddressSanitizer
# on its host code only (the device code of that file is unchanged), linked
# with the kernels' objects and a driver that exercises every host-side
# check without a GPU.
ASAN_HOST = "-Xarch_host -fsanitize=address -Xarch_host -fno-omit-frame-pointer".split()


def build_host_check(out_dir: str, driver: str) -> str:
    """Build the AddressSanitizer host check of the ABI layer into out_dir and
    return the executable's path. The kernels' objects come from _build/ (the
    library is built first when they are missing)."""
    os.makedirs(out_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    kernel_objs = [os.path.join(BUILD, os.path.basename(s) + ".o") for s in sources
                   if os.path.basename(s) != "abi.hip"]
    if not all(os.path.exists(o) for o in kernel_objs):
        build(verbose=False)
    flags = ["-O1", "-g", "-std=c++17", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC] + DEVICE_FLAGS
    abi_obj = os.path.join(out_dir, "abi_asan.o")
    drv_obj = os.path.join(out_dir, "driver_asan.o")
    exe = os.path.join(out_dir, "abi_host_check")
    steps = [
        [hipcc()] + flags + ASAN_HOST + ["-c", os.path.join(CSRC, "abi.hip"), "-o", abi_obj],
        [hipcc()] + flags + ASAN_HOST + ["-x", "hip", "-c", driver, "-o", drv_obj],
        [hipcc(), f"--offload-arch={ARCH}"] + ASAN_HOST + ["-o", exe, drv_obj, abi_obj] + kernel_objs,
    ]
    for cmd in steps:
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"host check build failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return exe


if __name__ == "__main__":
    build()
