"""A seeded sweep of decode steps (Jet-Long §3.2 Eqs. 4-5: the query at
position L-1 over L cached keys, read under G(L) and corrected as they are
read) against the float64 oracle, each also over the same cache held in
shuffled pages, which must agree bit for bit.  The draws cross GQA ratios
1-8, one to eight KV heads, D = 64 and 128, batches of one to three, page
sizes 32-512, G from 1 to over a hundred and lengths from a single key to
past 16K (many splits, ragged last steps).  Cache rows past L hold NaN."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
from gpu_common import TOL_BF16, max_err, require_gpu, to_dev
from test_gpu_paged import _paginate
import zero_shot_rope_jl_amd as jl

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=4242):
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        Hkv, R = int(rng.choice([1, 2, 4, 8])), int(rng.choice([1, 2, 4, 8]))
        Hq, D, B = Hkv * R, int(rng.choice([64, 128])), int(rng.integers(1, 4))
        # half the lengths short (down to a single key), half long (many splits)
        L = int(np.exp(rng.uniform(0, np.log(2000)))) if rng.random() < 0.5 else int(rng.integers(2000, 20001))
        if Hq > 32 or B * L * Hkv * D > 3e7:
            continue
        # one draw in five within the pretrained window (G = 1); the rest
        # w_pretrained log-uniform over [16, L]
        if rng.random() < 0.2:
            w_pre = L + int(rng.integers(0, 64))
        else:
            w_pre = int(np.exp(rng.uniform(np.log(16), np.log(max(L, 17)))))
        w0 = int(rng.integers(0, 800))
        ps = int(rng.choice([32, 64, 256, 512]))
        out.append((B, L, L + int(rng.integers(0, 70)), Hq, Hkv, D, w_pre, w0, ps))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES,
                         ids=[f"B{c[0]}_L{c[1]}_H{c[3]}x{c[4]}_D{c[5]}_wp{c[6]}_w0{c[7]}_ps{c[8]}" for c in CASES])
def test_decode_sweep_matches_oracle_and_paged(case):
    require_gpu()
    B, L, Lmax, Hq, Hkv, D, w_pre, w0, ps = case
    rng = np.random.Generator(np.random.PCG64([L, Hq, D, w0]))
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    qb, kb, vb = bits((B, 1, Hq, D)), bits((B, L, Hkv, D)), bits((B, L, Hkv, D))
    q = to_dev(qb, "bf16")
    kc = torch.full((B, Lmax, Hkv, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    kc[:, :L], vc[:, :L] = to_dev(kb, "bf16"), to_dev(vb, "bf16")
    base, scale = 1e4, D ** -0.5
    table = jl.alloc_table(Lmax, D, base, w_pretrained=w_pre)
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode(q, kc, vc, out, lse, L, w0, w_pre, base, scale, table, ws)
    kp, vp, bt = _paginate(kc, vc, ps, seed=L + ps)
    pout, plse = torch.empty_like(out), torch.empty_like(lse)
    jl.jl_bifocal_decode_paged(q, kp, vp, bt, pout, plse, L, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    f64 = lambda a: si.f32_from_bf16_bits(a).astype(np.float64)
    ref, ref_lse = oracle.decode_attention(f64(qb)[:, 0], f64(kb), f64(vb), L, w0, w_pre, base, scale)
    e, el = max_err(out.cpu().numpy()[:, 0], ref), max_err(lse.cpu().numpy(), ref_lse)
    print(case, "G", oracle.group_size(L, w_pre), "err", e, "lse", el)
    assert e <= TOL_BF16 and el <= TOL_BF16
    assert torch.equal(pout, out) and torch.equal(plse, lse)
