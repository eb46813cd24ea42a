"""The build's launch guard, checked on the CPU (nothing here runs on a GPU):
a kernel whose full workgroup cannot fit one compute unit -- its waves on a
SIMD need more than the 512 registers per lane the SIMD has, or it asks for
more than 160 KiB of LDS -- is found in the compiler's metadata and fails
the build, while kernels that fit pass."""
import importlib.util
import os
import shutil

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
spec = importlib.util.spec_from_file_location("_jl_build", os.path.join(ROOT, "zero_shot_rope_jl_amd", "build.py"))
build = importlib.util.module_from_spec(spec)
spec.loader.exec_module(build)

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="needs hipcc")

SRC = r"""
#include <hip/hip_runtime.h>
// 512 threads = 8 waves = 2 per SIMD; the clobber of register a255 forces
// the full 512 unified registers per wave: 2 x 512 > 512
__global__ __launch_bounds__(512) void too_many_regs(float* x) {
    asm volatile("" ::: "a255");
    x[threadIdx.x] += 1.f;
}
// the same clobber with one wave per SIMD fits
__global__ __launch_bounds__(256) void fits_regs(float* x) {
    asm volatile("" ::: "a255");
    x[threadIdx.x] += 1.f;
}
__global__ __launch_bounds__(256) void fits_lds(float* x) {
    __shared__ float s[40960];
    s[threadIdx.x * 160] = x[threadIdx.x];
    __syncthreads();
    x[threadIdx.x] = s[(255 - threadIdx.x) * 160];
}
"""


def test_guard_rejects_kernels_that_cannot_launch(tmp_path):
    src = tmp_path / "toy.hip"
    src.write_text(SRC)
    co = build.device_code_object(str(src), str(tmp_path / "toy.co"), [])
    ks = {k["name"]: k for k in build.kernel_resources(co)}
    names = {n.split("(")[0]: n for n in ks}
    by = {short: ks[full] for short, full in
          ((s, next(n for n in ks if s in n)) for s in ("too_many_regs", "fits_regs", "fits_lds"))}
    assert by["too_many_regs"]["agprs"] == 256 and by["too_many_regs"]["max_threads"] == 512
    assert by["fits_lds"]["lds"] == 40960 * 4
    bad = build.resource_violations(list(ks.values()))
    assert len(bad) == 1 and "too_many_regs" in bad[0]
    with pytest.raises(RuntimeError, match="cannot launch"):
        build.check_resources([co])
    assert names


def test_guard_rejects_lds_beyond_the_cu():
    """Static LDS beyond 160 KiB is already a compile error; the guard also
    catches it from the metadata (e.g. a kernel built by another route)."""
    k = {"name": "k", "max_threads": 256, "regs": 32, "lds": 160 * 1024 + 4}
    assert build.resource_violations([k]) and not build.resource_violations([dict(k, lds=160 * 1024)])


def test_library_kernels_fit():
    """Every kernel of the library as built here passes the guard."""
    objs = [os.path.join(build.BUILD, f) for f in os.listdir(build.BUILD)] if os.path.isdir(build.BUILD) else []
    cos = [o for o in objs if o.endswith(f".{build.ARCH}.co")]
    if not cos:
        pytest.skip("library not built")
    ks = build.check_resources(cos)
    assert any("prefill_bf16_kernel" in k["name"] for k in ks)
