"""Build libjetlong.so (gfx950) in-tree with hipcc.

    python -m zero_shot_rope_jl_amd.build [-v]

Every source under csrc/ is compiled to an object in _build/ (in parallel)
and linked into zero_shot_rope_jl_amd/libjetlong.so.  The compile line turns
off packed-FP32 code generation for the device and hides every symbol except
the C ABI declared in include/jetlong.h.  Sources listed in PER_FILE_FLAGS get
extra device-compiler options.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libjetlong.so")
ARCH = os.environ.get("JL_OFFLOAD_ARCH", "gfx950")
# The bf16 prefill keeps its score tiles, output accumulators and operands
# together within the 256 registers a wave has at two waves per SIMD; in the
# MFMAs' VGPR form (result and accumulator in ordinary VGPRs) the scores feed
# the exponentials directly, where the accumulation-register form would copy
# every score tile out of AGPRs and shuffle the accumulators between loop
# iterations.
PER_FILE_FLAGS = {"prefill_bf16.hip": ["-mllvm", "--amdgpu-mfma-vgpr-form"]}


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libjetlong.so)")


def compile_flags() -> list[str]:
    return [
        "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
        f"--offload-arch={ARCH}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", CSRC,
        "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas",
    ]


def _run(cmd: list[str], verbose: bool) -> None:
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(f for f in os.listdir(CSRC) if f.endswith(".hip"))
    cc = hipcc()
    flags = compile_flags()
    objs = []
    jobs = []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        for s in srcs:
            obj = os.path.join(BUILD, s[:-4] + ".o")
            objs.append(obj)
            extra = PER_FILE_FLAGS.get(s, [])
            jobs.append(ex.submit(_run, [cc, *flags, *extra, "-c", os.path.join(CSRC, s), "-o", obj], verbose))
        for j in jobs:
            j.result()
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
