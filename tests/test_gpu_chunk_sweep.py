"""A seeded sweep of chunk calls (Jet-Long §3.1 Eq. 2 with §3.2 Eqs. 4-5: Lq
new tokens over a cache of L keys are the last Lq rows of the prefill over
L tokens, under G(L)) against the float64 oracle rows.  The draws cross
both routes (the decode kernels for at most 64 position x query-head
columns per KV head, the prefill kernels otherwise), split and unsplit
query tiles, chunk lengths that leave the last query tile partly past L,
GQA ratios 1-8, D = 64 and 128, batches of one and two, and G from 1 to
85.  Cache rows past L hold NaN."""
import numpy as np
import pytest
import torch

import oracle
from gpu_common import TOL_BF16, max_err, require_gpu
from test_gpu_chunk import _run_chunk, _workload

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        Hkv, R = int(rng.choice([1, 2, 8])), int(rng.choice([1, 2, 4, 8]))
        Hq, D, B = Hkv * R, int(rng.choice([64, 128])), int(rng.choice([1, 2]))
        L = int(rng.integers(600, 12001))
        # half the draws short enough for the decode kernels
        short = rng.random() < 0.5
        Lq = int(rng.integers(1, (64 // R if short else min(L, 400)) + 1))
        if Hq > 16 or B * Lq * L * Hq > 6e7:
            continue
        # w_pretrained log-uniform over [64, 2L]: G = 1 up to G ~ L / 64
        w_pre = int(np.exp(rng.uniform(np.log(64), np.log(2 * L))))
        w0 = int(rng.integers(0, 601))
        out.append((B, L, Lq, L + int(rng.integers(0, 65)), Hq, Hkv, D, w_pre, w0))
    return out


CASES = _cases()


def _route(B, L, Lq, Hq, Hkv):
    """Which kernels the library picks (for the log): the decode kernels, or
    the prefill kernels with their key split count."""
    R = Hq // Hkv
    if Lq * R <= 64 and B * Lq <= 65535:
        return "decode kernels"
    wgs = -(-Lq // (256 // R)) * Hkv * B
    tiles = -(-L // 128)
    s = 1 if wgs >= 128 or tiles < 8 else max(1, min(256 // wgs, tiles // 4, 64))
    return f"prefill kernels, {s} split(s)"


@pytest.mark.parametrize("case", CASES,
                         ids=[f"B{c[0]}_L{c[1]}_Lq{c[2]}_H{c[4]}x{c[5]}_D{c[6]}_wp{c[7]}_w0{c[8]}" for c in CASES])
def test_chunk_sweep_matches_oracle(case):
    require_gpu()
    B, L, Lq, Lmax, Hq, Hkv, D, w_pre, w0 = case
    w = _workload(L, Hq, Hkv, D, w_pre, w0, B=B, seed=7 * L + Lq)
    x, out, lse = _run_chunk(w, Lq, Lmax, torch.float32)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale,
                                            rows=np.arange(L - Lq, L))
    o, s = out.cpu().numpy(), lse.cpu().numpy()
    e, el = max_err(o, ref), max_err(s, ref_lse)
    print(case, "G", oracle.group_size(L, w_pre), _route(B, L, Lq, Hq, Hkv), "err", e, "lse", el)
    assert np.all(np.isfinite(o))
    assert e <= TOL_BF16 and el <= TOL_BF16
