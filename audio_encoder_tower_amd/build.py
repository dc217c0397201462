"""Build libaenc.so (the HIP kernels and their C ABI) for gfx950 with hipcc.

Usage: python -m audio_encoder_tower_amd.build [--jobs N] [--debug] [--sanitize]

Each .hip source under csrc/ is compiled to an object in _build/, then the
objects are linked into audio_encoder_tower_amd/libaenc.so. No GPU is needed:
hipcc cross-compiles for gfx950.

--sanitize builds a separate copy, _build/sanitize/libaenc_sanitize.so, whose
host code (validation, the runtime, the cache bookkeeping) is instrumented
with AddressSanitizer and UndefinedBehaviorSanitizer; the device code is the
same. It is for host-side tests only: load it with the sanitizer runtime
preloaded and AENC_LIBRARY pointing at it.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libaenc.so")
ARCH = "gfx950"

# Packed fp32 VALU instructions are turned off on purpose: plain scalar fp32
# code is generated instead of v_pk_{add,mul,fma}_f32.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                # let the fully unrolled GEMM epilogues keep every accumulator in registers
                "-mllvm", "-pragma-unroll-threshold=200000"]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Host-only sanitizers (each -fsanitize= applies to the host pass alone).
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
SANITIZE_DIR = os.path.join(BUILD, "sanitize")
SANITIZE_LIB = os.path.join(SANITIZE_DIR, "libaenc_sanitize.so")

# Per-source extra device flags. The attention kernel's softmax works on the
# MFMA results directly, so they are kept in VGPRs rather than the AGPR file.
SOURCE_FLAGS = {"attention.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def compile_one(src: str, debug: bool, sanitize: bool = False) -> str:
    obj = os.path.join(SANITIZE_DIR if sanitize else BUILD, os.path.basename(src)[:-4] + ".o")
    opt = SANITIZE_FLAGS if sanitize else ["-O1" if debug else "-O3"]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-std=c++17", "-fPIC", "-c", src, "-o", obj,
           "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")] + opt
    cmd += DEVICE_FLAGS + SOURCE_FLAGS.get(os.path.basename(src), [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device feature flag above and says so.
    noise = "'-packed-fp32-ops' is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 8, debug: bool = False, sanitize: bool = False) -> str:
    os.makedirs(SANITIZE_DIR if sanitize else BUILD, exist_ok=True)
    srcs = sources()
    with ThreadPoolExecutor(max(1, jobs)) as pool:
        objs = list(pool.map(lambda s: compile_one(s, debug, sanitize), srcs))
    lib = SANITIZE_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    # a sanitized shared library leaves the sanitizer runtime to the process
    # (preloaded), so only the host pass is told about it
    link_extra = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"] if sanitize else []
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + link_extra + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, lib)
    return lib


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    ap.add_argument("--debug", action="store_true")
    ap.add_argument("--sanitize", action="store_true", help="host ASan + UBSan copy for host-side tests")
    args = ap.parse_args()
    print(build(args.jobs, args.debug, args.sanitize))


if __name__ == "__main__":
    main()
