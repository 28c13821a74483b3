"""Build libmxq.so (hand-written HIP for gfx950) in-tree, next to this file.

    python -m float8_quantization_moe_amd.build

Every source is compiled by hipcc for gfx950 only.  Packed fp32 VALU forms are
disabled for the device code (the kernels' fp32 arithmetic is plain scalar
multiply / med3 / convert).  Division stays correctly rounded (hipcc's default),
and denormals are not flushed.
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmxq.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

SOURCES = ["api.hip", "mx_codec.hip", "mx_dim0.hip", "dispatch.hip", "group_scale.hip", "group_split.hip", "transpose.hip",
           "grouped_mm.hip"]
ARCH = "gfx950"
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                "-Wno-unused-parameter", f"-I{os.path.join(ROOT, 'include')}"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: ROCm is required to build libmxq")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag and says so; that is harmless
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l and l.strip()]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build(verbose: bool = True) -> str:
    """Compile every HIP source and link libmxq.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


def build_host_asan(out_dir: str) -> str:
    """libmxq with AddressSanitizer on the host code (device code as usual), for
    the CPU tests of the C ABI's argument handling.  The sanitizer applies to the
    host pass only (-Xarch_host); load the result with the ASan runtime preloaded."""
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]

    def one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc(), *COMMON_FLAGS, *DEVICE_FLAGS, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (host ASan) failed for {src}:\n{res.stderr[-2000:]}")
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(one, SOURCES))
    out = os.path.join(out_dir, "libmxq_host_asan.so")
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
                    *objs, "-o", out], check=True)
    return out


if __name__ == "__main__":
    build()
