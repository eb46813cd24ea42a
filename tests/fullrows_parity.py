"""Every-row parity of a whole-sequence prefill at a full workload size:
the GPU computes the call once with bf16 and once with fp32 outputs, and the
float64 oracle (Jet-Long §3 Eq. 1 with the §3.3 Eq. 6 merge, §3.1 Eq. 3 /
§3.2 Eq. 5, over every causal key of a row) recomputes every query row of
every head, in 32 slices of equal work whose errors are printed as they
finish.  Bounds as in the GPU tests: max-abs 2e-2 on fp32 outputs and
log-sum-exps, and on bf16 outputs (elements with |ref| >= 4 may add the
half-ulp rounding of the exact value).

Not collected by pytest (the oracle takes ~10 min for the 64K workload on
16 host cores); run on a GPU host from the repository root:

    python tests/fullrows_parity.py ext64k

Exits non-zero if any slice exceeds a bound."""
import os
import sys
import time

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path[:0] = [HERE, os.path.dirname(HERE)]

import synth_inputs as si  # noqa: E402
import zero_shot_rope_jl_amd as jl  # noqa: E402
from gpu_common import (TOL_BF16, assert_bf16_out_close, max_err, oracle_rows_parallel, prefill,  # noqa: E402
                        require_gpu, to_dev)


def main(name: str) -> int:
    require_gpu()
    w = si.WORKLOADS[name]
    t0 = time.perf_counter()
    print(f"[fullrows] {name}: B{w.B} L{w.L} Hq{w.Hq} Hkv{w.Hkv} D{w.D} w0 {w.w0} w_pretrained {w.w_pretrained}",
          flush=True)
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    got = {}
    for od in (torch.bfloat16, torch.float32):
        out, lse = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, od, table)
        got[od] = (out.float().cpu().numpy(), lse.cpu().numpy())
        del out, lse
    del q, k, v
    torch.cuda.empty_cache()
    q64 = si.f32_from_bf16_bits(x["q"]).astype(np.float64)
    k64 = si.f32_from_bf16_bits(x["k"]).astype(np.float64)
    v64 = si.f32_from_bf16_bits(x["v"]).astype(np.float64)
    print(f"[fullrows] GPU outputs and float64 inputs ready ({time.perf_counter() - t0:.0f} s)", flush=True)
    rows = np.arange(w.L, dtype=np.int64)
    cost = np.cumsum(rows.astype(np.float64) + 1.0)
    cuts = np.searchsorted(cost, cost[-1] * np.arange(1, 32) / 32)
    worst = {"fp32": 0.0, "bf16": 0.0, "lse": 0.0}
    ok = True
    for i, part in enumerate(np.split(rows, cuts)):
        ref, ref_lse = oracle_rows_parallel(q64, k64, v64, part, w.w0, w.w_pretrained, w.rope_base, w.sm_scale)
        e32 = max_err(got[torch.float32][0][:, part], ref)
        el = max_err(got[torch.float32][1][:, :, part], ref_lse)
        try:
            e16, _ = assert_bf16_out_close(got[torch.bfloat16][0][:, part], ref, label=f"{name} slice {i}")
        except AssertionError as exc:
            print(f"[fullrows] slice {i}: {exc}", flush=True)
            e16, ok = float("inf"), False
        ok = ok and e32 <= TOL_BF16 and el <= TOL_BF16
        for key, e in (("fp32", e32), ("bf16", e16), ("lse", el)):
            worst[key] = max(worst[key], e)
        print(f"[fullrows] slice {i + 1}/32 rows {part[0]}..{part[-1]}: fp32-out {e32:.3e} bf16-out {e16:.3e} "
              f"lse {el:.3e} ({time.perf_counter() - t0:.0f} s)", flush=True)
    print(f"[fullrows] {name}: all {w.L} rows x {w.Hq} heads x {w.B} sequence(s): max err fp32-out {worst['fp32']:.3e}, "
          f"bf16-out {worst['bf16']:.3e}, lse {worst['lse']:.3e}; bound {TOL_BF16}: {'ok' if ok else 'EXCEEDED'} "
          f"({time.perf_counter() - t0:.0f} s)", flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main(sys.argv[1] if len(sys.argv) > 1 else "ext64k"))
