"""Helpers shared by the GPU tests: device tensors from the seeded inputs and
thin wrappers that call the library through its C ABI binding."""
import numpy as np
import torch

import zero_shot_rope_jl_amd as jl

TOL_BF16 = 2e-2      # max-abs bound for bf16 inputs
TOL_F32 = 1e-5       # max-abs bound for fp32 inputs
BF16_HALF_ULP_REL = 2.0 ** -8   # rounding an exact value to bf16 moves it by <= this * |value|


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch.device("cuda")


def to_dev(arr, dtype):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    return t.cuda()


def prefill(q, k, v, w0, w_pre, base, scale, out_dtype, table=None, with_lse=True):
    B, L, Hq, D = q.shape
    if table is None:
        table = jl.alloc_table(L, D, base)
    out = torch.empty((B, L, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device=q.device) if with_lse else None
    jl.jl_bifocal_prefill(q, k, v, out, lse, w0, w_pre, base, scale, table)
    torch.cuda.synchronize()
    return out, lse


def max_err(got, want):
    return float(np.max(np.abs(np.asarray(got, np.float64) - np.asarray(want, np.float64))))


def assert_bf16_out_close(got, want, tol=TOL_BF16):
    """bf16 output: the error budget is the bound plus the unavoidable
    rounding of the exact result to bf16."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    excess = np.abs(got - want) - (tol + BF16_HALF_ULP_REL * np.abs(want))
    assert np.all(excess <= 0), f"max excess {excess.max():.3g} (max abs err {max_err(got, want):.3g})"
