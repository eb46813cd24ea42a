"""Whole-sequence bf16 prefills large enough for the bf16 kernel's dynamic
grid (one workgroup per compute unit taking query tiles from per-XCD queues,
used when the one-workgroup-per-tile grid would take more than two rounds),
over shapes that mix batches and KV heads in the queues: batches of two and
three, two to eight KV heads, D = 64 and 128, G = 1 and G > 1, and lengths
that leave the last query tile ragged.  Each is compared with the float64
oracle (Jet-Long §3 Eq. 1 with the §3.3 Eq. 6 merge, §3.1 Eq. 3 / §3.2 Eq. 5)
on sampled rows: 48 seeded rows, the first and last 16, and the rows next
to the multiples of w0 + 1 and w_pretrained."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_common import TOL_BF16, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu

#        B      L   Hq Hkv   D  w_pre    w0
CASES = [(2, 17000, 8, 2, 128, 4500, 700),
         (1, 20000, 16, 4, 64, 3000, 300),
         (3, 9000, 8, 8, 128, 2000, 1000),
         (1, 24000, 32, 8, 128, 24000, 100)]


def _rows(L, w0, w_pre, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(rng.integers(0, L, 48).tolist()) | set(range(16)) | set(range(L - 16, L))
    for step in (w0 + 1, w_pre):
        for m in range(step, L, step):
            rows |= {r for r in (m - 1, m, m + 1) if 0 <= r < L}
    return np.array(sorted(rows))


@pytest.mark.parametrize("case", CASES,
                         ids=[f"B{c[0]}_L{c[1]}_H{c[2]}x{c[3]}_D{c[4]}_wp{c[5]}_w0{c[6]}" for c in CASES])
def test_dynamic_grid_prefill_matches_oracle_rows(case):
    require_gpu()
    B, L, Hq, Hkv, D, w_pre, w0 = case
    BQ = 256 // (Hq // Hkv)
    n_tiles = -(-L // BQ) * Hkv * B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[dynamic grid] case {case}: {n_tiles} query tiles over {n_cu} compute units", flush=True)
    assert n_tiles > 2 * n_cu, "the case must take the dynamic grid"
    w = si.Workload(f"dyn{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, 5 * L + Hq)
    x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    out, lse = prefill(q, k, v, w0, w_pre, w.rope_base, w.sm_scale, torch.float32)
    rows = _rows(L, w0, w_pre, L)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale,
                                            rows=rows)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    e = max_err(o[:, rows], ref)
    el = max_err(lse.cpu().numpy()[:, :, rows], ref_lse)
    print(f"[dynamic grid] G {oracle.group_size(L, w_pre)} rows {len(rows)} err {e:.3e} lse {el:.3e}", flush=True)
    assert e <= TOL_BF16 and el <= TOL_BF16
