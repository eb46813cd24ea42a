"""GPU parity of jl_bifocal_decode_paged: a decode step over a cache held in
shuffled fixed-size pages equals the same step over the contiguous cache
(Jet-Long §3.2 Eqs. 4-5: the cached keys are read as stored and corrected on
the fly, wherever they sit), and the float64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _cache(B, Lmax, Hkv, D, seed):
    rng = np.random.Generator(np.random.PCG64([seed, 3]))
    kb = si.bf16_bits_from_f32(rng.standard_normal((B, Lmax, Hkv, D), dtype=np.float32))
    vb = si.bf16_bits_from_f32(rng.standard_normal((B, Lmax, Hkv, D), dtype=np.float32))
    qb = si.bf16_bits_from_f32(rng.standard_normal((B, 1, 4 * Hkv, D), dtype=np.float32))
    return qb, kb, vb


def _paginate(kc, vc, page_size, seed, spare=3):
    """Pages in a shuffled order (plus unused pages) and the block table."""
    B, Lmax, Hkv, D = kc.shape
    max_pages = (Lmax + page_size - 1) // page_size
    n_pages = B * max_pages + spare
    perm = np.random.Generator(np.random.PCG64([seed, 5])).permutation(n_pages)[: B * max_pages]
    kp = torch.zeros((n_pages, page_size, Hkv, D), dtype=kc.dtype, device=kc.device)
    vp = torch.zeros_like(kp)
    for b in range(B):
        for s in range(max_pages):
            pg = int(perm[b * max_pages + s])
            rows = slice(s * page_size, min((s + 1) * page_size, Lmax))
            n = rows.stop - rows.start
            kp[pg, :n] = kc[b, rows]
            vp[pg, :n] = vc[b, rows]
    bt = torch.from_numpy(perm.reshape(B, max_pages).astype(np.int32)).to(kc.device)
    return kp, vp, bt


CASES = [  # (B, L, Lmax, Hkv, D, page_size, w_pre, w0)
    (2, 1537, 1600, 2, 128, 64, 400, 100),
    (1, 100, 130, 2, 64, 32, 64, 10),
    (2, 20000, 20050, 2, 128, 256, 4096, 512),   # many splits, G = 5
    (1, 1, 40, 8, 128, 32, 16, 0),
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_L{c[1]}_Hkv{c[3]}_D{c[4]}_ps{c[5]}" for c in CASES])
def test_paged_equals_contiguous_and_oracle(case):
    require_gpu()
    B, L, Lmax, Hkv, D, ps, w_pre, w0 = case
    Hq, base, scale = 4 * Hkv, 1e4, D ** -0.5
    qb, kb, vb = _cache(B, Lmax, Hkv, D, seed=L)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_workspace(B, Hq, D, L)
    ref_out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    ref_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode(q, kc, vc, ref_out, ref_lse, L, w0, w_pre, base, scale, table, ws)
    kp, vp, bt = _paginate(kc, vc, ps, seed=L + ps)
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    jl.jl_bifocal_decode_paged(q, kp, vp, bt, out, lse, L, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    f64 = lambda a: si.f32_from_bf16_bits(a).astype(np.float64)
    dref, dref_lse = oracle.decode_attention(f64(qb)[:, 0], f64(kb), f64(vb), L, w0, w_pre, base, scale)
    e, el = max_err(out.cpu().numpy()[:, 0], dref), max_err(lse.cpu().numpy(), dref_lse)
    print(case, "G", oracle.group_size(L, w_pre), "err", e, "lse", el)
    assert e <= TOL_BF16 and el <= TOL_BF16


def test_out_of_range_page_poisons_only_its_sequence():
    require_gpu()
    B, L, Lmax, Hkv, D, ps = 2, 700, 768, 2, 128, 64
    Hq, base, scale, w_pre, w0 = 4 * Hkv, 1e4, D ** -0.5, 256, 64
    qb, kb, vb = _cache(B, Lmax, Hkv, D, seed=77)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_workspace(B, Hq, D, L)
    kp, vp, bt = _paginate(kc, vc, ps, seed=78)
    good = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode_paged(q, kp, vp, bt, good, None, L, w0, w_pre, base, scale, table, ws)
    bad_bt = bt.clone()
    bad_bt[1, 3] = kp.shape[0] + 1000      # past the last page
    bad_bt[1, 5] = -7
    out = torch.empty_like(good)
    jl.jl_bifocal_decode_paged(q, kp, vp, bad_bt, out, None, L, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    assert torch.equal(out[0], good[0])
    assert torch.isnan(out[1]).all()
