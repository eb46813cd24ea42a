"""Build libjetlong.so (gfx950) in-tree with hipcc.

    python -m zero_shot_rope_jl_amd.build [-v]

Every source under csrc/ is compiled to an object in _build/ (in parallel)
and linked into zero_shot_rope_jl_amd/libjetlong.so.  The device side of each
source is also compiled alone, and the build fails if the metadata of any
kernel shows a workgroup that cannot fit one compute unit (registers times
the waves each SIMD must hold, or LDS).  The compile line turns
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


# Per-CU limits of gfx950 that a launch must fit: each SIMD has 512 unified
# registers (VGPRs and AGPRs) per lane for its resident waves, a workgroup's
# waves are spread over the CU's 4 SIMDs, and a workgroup may use up to
# 160 KiB of LDS.
REGS_PER_SIMD_LANE = 512
REG_GRANULE = 8
SIMDS_PER_CU = 4
LDS_BYTES_PER_CU = 160 * 1024


def kernel_resources(code_object: str) -> list[dict]:
    """Per-kernel resource usage recorded by the compiler in a device code
    object's metadata notes (llvm-readelf --notes): name, the maximum
    workgroup size the kernel is compiled for (from __launch_bounds__),
    unified register count (VGPRs + AGPRs), AGPRs, LDS bytes, spills."""
    readelf = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", "llvm-readelf")
    r = subprocess.run([readelf, "--notes", code_object], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"llvm-readelf failed on {code_object}: {r.stderr}")
    fields = {".name": "name", ".max_flat_workgroup_size": "max_threads", ".vgpr_count": "regs",
              ".agpr_count": "agprs", ".group_segment_fixed_size": "lds", ".vgpr_spill_count": "vgpr_spills",
              ".sgpr_spill_count": "sgpr_spills", ".private_segment_fixed_size": "scratch"}
    kernels, cur = [], None
    for line in r.stdout.splitlines():
        t = line.strip()
        if t.startswith("- "):          # a new entry of the .kernels list
            t = t[2:].strip()
            if t.startswith(".agpr_count") or t.startswith(".args") or t.startswith(".name"):
                cur = {}
                kernels.append(cur)
        if cur is None or ":" not in t:
            continue
        key, _, val = t.partition(":")
        if key in fields:
            val = val.strip()
            cur[fields[key]] = val if key == ".name" else int(val)
    return [k for k in kernels if "name" in k and "regs" in k]


def resource_violations(kernels: list[dict]) -> list[str]:
    """Kernels whose launch cannot fit one CU: the waves of a full workgroup
    placed on a SIMD need more registers than it has, or the LDS exceeds the
    CU's.  Such a launch aborts at dispatch instead of running."""
    bad = []
    for k in kernels:
        waves = -(-k.get("max_threads", 1024) // 64)
        per_simd = -(-waves // SIMDS_PER_CU)
        regs = -(-k["regs"] // REG_GRANULE) * REG_GRANULE
        if regs * per_simd > REGS_PER_SIMD_LANE:
            bad.append(f"{k['name']}: {regs} registers x {per_simd} waves per SIMD "
                       f"(workgroup of {k.get('max_threads')} threads) > {REGS_PER_SIMD_LANE}")
        if k.get("lds", 0) > LDS_BYTES_PER_CU:
            bad.append(f"{k['name']}: {k['lds']} bytes of LDS > {LDS_BYTES_PER_CU}")
    return bad


def device_code_object(src: str, out: str, extra: list[str], verbose: bool = False) -> str:
    """Compile the device side of one source alone into a code object."""
    _run([hipcc(), *compile_flags(), *extra, "--offload-device-only", "--no-gpu-bundle-output", "-c", src,
          "-o", out], verbose)
    return out


def check_resources(code_objects: list[str]) -> list[dict]:
    kernels = [k for co in code_objects for k in kernel_resources(co)]
    bad = resource_violations(kernels)
    if bad:
        raise RuntimeError("kernels that cannot launch on gfx950:\n  " + "\n  ".join(bad))
    return kernels


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
            # a fixed compilation-unit id: by default hipcc hashes it from the
            # source path, so the same sources built in another directory gave
            # a library with other bytes
            cuid = f"-cuid=jl_{s[:-4]}"
            jobs.append(ex.submit(_run, [cc, *flags, *extra, cuid, "-c", os.path.join(CSRC, s), "-o", obj], verbose))
        cos = [ex.submit(device_code_object, os.path.join(CSRC, s), os.path.join(BUILD, s[:-4] + f".{ARCH}.co"),
                         PER_FILE_FLAGS.get(s, []), verbose) for s in srcs]
        for j in jobs:
            j.result()
        # every kernel must fit a CU at the workgroup size it is compiled for
        kernels = check_resources([c.result() for c in cos])
    if verbose:
        for k in kernels:
            print(f"{k['regs']:4d} regs ({k.get('agprs', 0):3d} AGPR) {k.get('lds', 0):7d} B LDS "
                  f"{k.get('max_threads')} threads  {k['name']}")
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
