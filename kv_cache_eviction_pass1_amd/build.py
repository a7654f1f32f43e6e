"""Build libdropkv.so (HIP, gfx950) in-tree with hipcc.

Every source under csrc/ is compiled for gfx950 only and linked into one
shared library next to this file. Packed-FP32 instruction selection is
disabled for device code.

Two checking variants are built next to it on request (never loaded unless
DROPKV_LIBRARY names them):
  --debug  libdropkv_debug.so: device-side bounds checks on the global
           indices of the scoring kernels (pass 1, merge, pass 2, select,
           compaction, prefill); a failed check raises DROPKV_STATUS_BOUNDS
           in the call's status word instead of trapping.
  --asan   libdropkv_asan.so: the host code of the C ABI (argument
           validation, workspace carving, dispatch) compiled with
           AddressSanitizer (host code only: -Xarch_host); load it with the
           clang ASan runtime preloaded (asan_runtime()).
"""

from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdropkv.so")
LIB_DEBUG = os.path.join(PKG, "libdropkv_debug.so")
LIB_ASAN = os.path.join(PKG, "libdropkv_asan.so")
ARCH = "gfx950"

DEVICE_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
    # Every global atomic here is issued by one lane. The compiler's atomic
    # optimizer would still rewrite a uniform-address atomic into a wave
    # reduction that waits for all outstanding memory operations right after
    # it (vmcnt(0)), draining the tile loads in flight behind a tile claim.
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
]
# host code of the C ABI under AddressSanitizer; device code is unchanged
ASAN_HOST_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
                   "-Xarch_host", "-g"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that matches hipcc (to LD_PRELOAD)."""
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    cands += sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang ASan runtime not found")
    return cands[-1]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build(verbose: bool = False, variant: str = "release") -> str:
    """Compile every HIP source for gfx950 and link the library; returns its path.

    variant: "release" (libdropkv.so), "debug" (bounds-checked kernels) or
    "asan" (host code under AddressSanitizer).
    """
    if variant not in ("release", "debug", "asan"):
        raise ValueError(variant)
    cc = hipcc()
    objdir = os.path.join(PKG, "_build" if variant == "release" else f"_build_{variant}")
    os.makedirs(objdir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        flags = list(DEVICE_FLAGS)
        if variant == "debug":
            flags.append("-DDROPKV_DEBUG=1")
        if variant == "asan":
            flags += ASAN_HOST_FLAGS
        cmd = [cc, *flags, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in res.stderr.splitlines()
                         if "packed-fp32-ops" not in l or "error" in l)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
        if verbose and errs.strip():
            print(errs, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, sources()))
    out = {"release": LIB, "debug": LIB_DEBUG, "asan": LIB_ASAN}[variant]
    tmp = out + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if variant == "asan":
        cmd[1:1] = ["-Xarch_host", "-fsanitize=address", "-shared-libasan"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    var = "debug" if "--debug" in sys.argv else ("asan" if "--asan" in sys.argv else "release")
    print(build(verbose="-v" in sys.argv, variant=var))
