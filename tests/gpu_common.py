"""Helpers shared by the GPU tests: device tensors from the seeded inputs,
thin wrappers that call the library through its C ABI binding, the parity
bounds, and a threaded driver that runs the float64 oracle over many query
rows (or decode steps) at once on the host's cores."""
import concurrent.futures as cf
import os

import numpy as np
import torch

import oracle
import zero_shot_rope_jl_amd as jl

TOL_BF16 = 2e-2      # max-abs bound for bf16 inputs
TOL_F32 = 1e-5       # max-abs bound for fp32 inputs
# A bf16 output cannot hold the exact result closer than half a bf16 ulp:
# 2^-9 relative, i.e. 0.0156 for |out| in [4, 8).  From |ref| >= 4 up that
# rounding alone can exceed part of the 2e-2 budget, so only there the bound
# is widened by it; every element below 4 is held to the plain 2e-2.
BF16_HALF_ULP_REL = 2.0 ** -8
BF16_WIDEN_FROM = 4.0


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


def assert_bf16_out_close(got, want, tol=TOL_BF16, label=""):
    """bf16 output against the oracle: max-abs <= tol on every element with
    |ref| < 4; elements with |ref| >= 4 may add the half-ulp rounding of the
    exact result to bf16.  Prints how many elements used the allowance and
    returns (max abs err, that count)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    big = np.abs(want) >= BF16_WIDEN_FROM
    n_big = int(big.sum())
    small_err = float(err[~big].max()) if n_big < err.size else 0.0
    assert small_err <= tol, f"{label} max abs err {small_err:.3g} on |ref| < {BF16_WIDEN_FROM} (bound {tol})"
    if n_big:
        excess = err[big] - (tol + BF16_HALF_ULP_REL * np.abs(want[big]))
        assert np.all(excess <= 0), f"{label} |ref| >= {BF16_WIDEN_FROM}: max excess {excess.max():.3g}"
        print(f"[parity] {label} {n_big} of {err.size} bf16-out elements have |ref| >= {BF16_WIDEN_FROM} "
              f"(max err there {float(err[big].max()):.3g}); plain-bound max err elsewhere {small_err:.3g}",
              flush=True)
    return float(err.max()), n_big


def host_workers():
    """Oracle worker threads: the cores this process may use, at most 16 (one
    GPU's share of a box's host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover
        import contextlib
        return contextlib.nullcontext()


def oracle_rows_parallel(q64, k64, v64, rows, w0, w_pre, base, scale, workers=None, fn=None):
    """oracle.bifocal_attention (or ``fn`` with its signature) over ``rows``,
    split into contiguous slices that run on separate threads with one BLAS
    thread each (NumPy releases the interpreter lock inside its kernels).
    Each slice is an ordinary oracle call on the same full-length inputs, so
    the result equals one call over all rows."""
    fn = fn or oracle.bifocal_attention
    rows = np.asarray(rows, dtype=np.int64)
    workers = workers or host_workers()
    # slices of ~equal work: a row costs ~ its key count
    cost = np.cumsum(rows.astype(np.float64) + 1.0)
    cuts = np.searchsorted(cost, cost[-1] * np.arange(1, 4 * workers) / (4 * workers))
    parts = [p for p in np.split(rows, np.unique(cuts)) if len(p)]
    with _one_blas_thread(), cf.ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda r: fn(q64, k64, v64, w0, w_pre, base, scale, rows=r), parts))
    return np.concatenate([o for o, _ in res], axis=1), np.concatenate([l for _, l in res], axis=2)


def oracle_decode_parallel(steps, k64, v64, w0, w_pre, base, scale, workers=None):
    """oracle.decode_attention for several steps of one cache: ``steps`` is a
    list of (q_tok [B, Hq, D] float64, L); step s reads rows < L of k64/v64.
    Returns a list of (out, lse) in the same order."""
    workers = workers or host_workers()
    with _one_blas_thread(), cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(lambda s: oracle.decode_attention(s[0], k64, v64, s[1], w0, w_pre, base, scale), steps))
