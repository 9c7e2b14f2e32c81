"""Build libautofp.so (HIP, gfx950) in-tree with hipcc.

    python -m runtime_mixed_precision_amd.build        # or build() from Python

Each translation unit under csrc/ is compiled in parallel into _build/, then
linked into runtime_mixed_precision_amd/libautofp.so.
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libautofp.so")
SOURCES = ["api.hip", "encode.hip", "gemv.hip", "gemv_batch.hip", "gemm.hip", "gptq.hip", "kv.hip", "signals.hip"]
ARCH = os.environ.get("AUTOFP_OFFLOAD_ARCH", "gfx950")

# Packed fp32 vector instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Per-source flags. kv.hip: MFMA accumulators in ordinary VGPRs, so the split
# kernel's output tile is not held twice (accumulation registers + VGPRs) and
# two wavefronts fit per SIMD.
SOURCE_FLAGS = {"kv.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Werror", "-Wno-unused-function", "-Wno-unused-command-line-argument"]


def hipcc():
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the AutoFP library needs ROCm's hipcc")


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side sanitizers for the C ABI's argument checks (api.hip's host code);
# each flag goes to the host compile only, device code is built as in build().
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]
SANITIZED_LIB = os.path.join(BUILD, "libautofp_hostsan.so")


def asan_runtime():
    """Path of clang's shared AddressSanitizer runtime (to preload into a
    process that loads the sanitized library), or None."""
    import glob
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for base in (os.path.join(root, "lib", "llvm"), os.path.join(root, "llvm"), "/opt/rocm/lib/llvm"):
        hits = sorted(glob.glob(os.path.join(base, "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
        if hits:
            return hits[-1]
    return None


def build_host_sanitized():
    """libautofp with api.hip's host code under AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the other objects of build()
    (run build() first): _build/libautofp_hostsan.so."""
    os.makedirs(BUILD, exist_ok=True)
    obj = os.path.join(BUILD, "api_hostsan.o")
    cmd = [hipcc(), *[c for c in COMMON if c != "-O3"], "-O1", "-g", *DEVICE_FLAGS, *HOST_SANITIZE, "-c",
           os.path.join(CSRC, "api.hip"), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on api.hip (host sanitizers):\n{res.stdout}\n{res.stderr}")
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES if src != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"run build() first: missing {missing}")
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-shared-libasan", obj, *objs, "-o", SANITIZED_LIB]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed (host sanitizers):\n{res.stdout}\n{res.stderr}")
    return SANITIZED_LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
