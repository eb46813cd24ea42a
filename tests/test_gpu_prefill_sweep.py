"""A seeded sweep of whole-sequence bf16 prefills (Jet-Long §3 Eq. 1 with the
§3.3 Eq. 6 merge, remote view of §3.1 Eq. 3 / §3.2 Eq. 5) against the
float64 oracle on sampled rows: 64 seeded rows, the first and last 32 and
the rows next to every multiple of w0 and w_pretrained in range.  The draws
cross GQA ratios 1-8, one to four KV heads, D = 64 and 128, batches of one
and two, G from 1 to the tens, and lengths that leave the last query tile
ragged (blocks of it wholly past L)."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_common import TOL_BF16, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=777):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        Hkv, R = int(rng.choice([1, 2, 4])), int(rng.choice([1, 2, 4, 8]))
        Hq, D, B = Hkv * R, int(rng.choice([64, 128])), int(rng.choice([1, 2]))
        L = int(rng.integers(33, 4001))
        if B * L * Hq * D > 2e7:
            continue
        w_pre = int(np.exp(rng.uniform(np.log(32), np.log(2 * L))))
        w0 = int(rng.integers(0, min(L, 700)))
        out.append((B, L, Hq, Hkv, D, w_pre, w0))
    return out


CASES = _cases()


def _rows(L, w0, w_pre, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = set(rng.integers(0, L, 64).tolist()) | set(range(min(32, L))) | set(range(max(0, L - 32), L))
    for step in (w0 + 1, w_pre):
        if step < 16:   # a window this small: its edges are in every sampled row's reach
            continue
        for m in range(step, L, step):
            rows |= {r for r in (m - 1, m, m + 1) if 0 <= r < L}
    return np.array(sorted(rows))


@pytest.mark.parametrize("case", CASES,
                         ids=[f"B{c[0]}_L{c[1]}_H{c[2]}x{c[3]}_D{c[4]}_wp{c[5]}_w0{c[6]}" for c in CASES])
def test_prefill_sweep_matches_oracle_rows(case):
    require_gpu()
    B, L, Hq, Hkv, D, w_pre, w0 = case
    w = si.Workload(f"sweep{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, 3 * L + Hq)
    x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    out, lse = prefill(q, k, v, w0, w_pre, w.rope_base, w.sm_scale, torch.float32)
    rows = _rows(L, w0, w_pre, L)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale,
                                            rows=rows)
    o = out.cpu().numpy()[:, rows]
    s = lse.cpu().numpy()[:, :, rows]
    e, el = max_err(o, ref), max_err(s, ref_lse)
    print(case, "G", oracle.group_size(L, w_pre), "rows", len(rows), "err", e, "lse", el)
    assert np.all(np.isfinite(out.cpu().numpy()))
    assert e <= TOL_BF16 and el <= TOL_BF16
