"""GPU parity of jl_bifocal_decode_rkc, decode with a rotated-key cache:
every remote key is read already in its remote view R(f(k) - k)·k (Jet-Long
§3.2 Eq. 5) from a cache the call keeps up to date, instead of being rotated
as it is read.  Checked against the float64 oracle, against the on-the-fly
decode, across a change of G (the cache is rebuilt), and for the cache's
own rows (incremental updates equal a fresh build)."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _cache(B, Lmax, Hq, Hkv, D, seed):
    rng = np.random.Generator(np.random.PCG64([seed, 13]))
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    return bits((B, 1, Hq, D)), bits((B, Lmax, Hkv, D)), bits((B, Lmax, Hkv, D))


def _f64(a):
    return si.f32_from_bf16_bits(a).astype(np.float64)


CASES = [  # (B, L, Lmax, Hq, Hkv, D, w_pre, w0)
    (2, 1537, 1600, 8, 2, 128, 400, 100),     # G = 4, window edge inside a 32-key step
    (1, 1000, 1100, 4, 2, 64, 300, 64),       # D = 64
    (1, 20000, 20050, 32, 8, 128, 4096, 1000),  # many splits, G = 5
    (1, 600, 700, 8, 8, 128, 256, 0),         # w0 = 0, no GQA
    (1, 300, 320, 16, 2, 128, 100, 400),      # w0 >= L: no remote key, the cache is not read
    (1, 400, 420, 8, 2, 128, 1000, 30),       # G = 1
    (2, 65, 70, 4, 2, 64, 1, 3),              # w_pretrained = 1: G = L
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_L{c[1]}_H{c[3]}x{c[4]}_D{c[5]}_wp{c[6]}_w0{c[7]}"
                                              for c in CASES])
def test_rkc_decode_matches_oracle_and_on_the_fly(case):
    require_gpu()
    B, L, Lmax, Hq, Hkv, D, w_pre, w0 = case
    base, scale = 1e4, D ** -0.5
    qb, kb, vb = _cache(B, Lmax, Hq, Hkv, D, seed=L + Hq)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    rkc = jl.RotatedKeyCache(kc)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode_rkc(q, kc, vc, rkc, out, lse, L, w0, w_pre, base, scale, table, ws)
    fly = torch.empty_like(out)
    fly_lse = torch.empty_like(lse)
    jl.jl_bifocal_decode(q, kc, vc, fly, fly_lse, L, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    G = oracle.group_size(L, w_pre)
    kloc = 0 if G == 1 else max(0, L - 1 - min(w0, L))
    if kloc > 0:   # the remote rows, and the first local row written ahead for the next step
        assert (rkc.state.G, rkc.state.rows) == (G, kloc + 1)
    else:
        assert (rkc.state.G, rkc.state.rows) == (0, 0)
    ref, ref_lse = oracle.decode_attention(_f64(qb)[:, 0], _f64(kb), _f64(vb), L, w0, w_pre, base, scale)
    e, el = max_err(out.cpu().numpy()[:, 0], ref), max_err(lse.cpu().numpy(), ref_lse)
    d = max_err(out.cpu().numpy(), fly.cpu().numpy())
    print(case, "G", G, "err", e, "lse", el, "vs on the fly", d)
    assert e <= TOL_BF16 and el <= TOL_BF16
    assert d <= TOL_BF16


def test_rkc_steps_across_a_change_of_g():
    """Steps L = 1530 .. 1541 with w_pretrained 512: G = 3 up to L = 1536,
    G = 4 from 1537 on.  The cache grows one row per step (written ahead by
    the decode kernel) and is rebuilt at the change; every step matches the
    oracle, and the rows built step by step equal a fresh build (the
    rotation kernel) bit for bit."""
    require_gpu()
    B, Lmax, Hq, Hkv, D, w_pre, w0, base = 1, 1600, 8, 2, 128, 512, 100, 1e4
    scale = D ** -0.5
    _, kb, vb = _cache(B, Lmax, Hq, Hkv, D, seed=5)
    kc, vc = to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    rkc = jl.RotatedKeyCache(kc)
    rng = np.random.Generator(np.random.PCG64([6, 1]))
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    prev_G = None
    for L in range(1530, 1542):
        qb = si.bf16_bits_from_f32(rng.standard_normal((B, 1, Hq, D), dtype=np.float32))
        jl.jl_bifocal_decode_rkc(to_dev(qb, "bf16"), kc, vc, rkc, out, None, L, w0, w_pre, base, scale, table, ws)
        torch.cuda.synchronize()
        G = oracle.group_size(L, w_pre)
        assert (rkc.state.G, rkc.state.rows) == (G, L - w0)
        ref, _ = oracle.decode_attention(_f64(qb)[:, 0], _f64(kb), _f64(vb), L, w0, w_pre, base, scale)
        e = max_err(out.cpu().numpy()[:, 0], ref)
        print("L", L, "G", G, "err", e, "rebuilt" if prev_G not in (None, G) else "")
        assert e <= TOL_BF16
        prev_G = G
    rows = rkc.state.rows
    fresh = jl.RotatedKeyCache(kc)
    jl.jl_bifocal_decode_rkc(to_dev(qb, "bf16"), kc, vc, fresh, out, None, 1541, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    assert fresh.state.rows == rows
    assert torch.equal(rkc.keys[:, :rows], fresh.keys[:, :rows])


def test_rkc_a_mismatched_table_poisons_until_reset():
    """A table built for another RoPE base: that step is NaN and so is the
    next one with the right table under the same G (4 for L = 700 .. 702;
    the cache rows it wrote are NaN); after a reset the steps match the
    oracle again."""
    require_gpu()
    B, Lmax, Hq, Hkv, D, w_pre, w0, base = 1, 900, 8, 2, 128, 200, 50, 1e4
    scale = D ** -0.5
    qb, kb, vb = _cache(B, Lmax, Hq, Hkv, D, seed=11)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    good, wrong = jl.alloc_table(Lmax, D, base), jl.alloc_table(Lmax, D, 5e5)
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    rkc = jl.RotatedKeyCache(kc)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode_rkc(q, kc, vc, rkc, out, None, 700, w0, w_pre, base, scale, wrong, ws)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    jl.jl_bifocal_decode_rkc(q, kc, vc, rkc, out, None, 701, w0, w_pre, base, scale, good, ws)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    rkc.reset()
    jl.jl_bifocal_decode_rkc(q, kc, vc, rkc, out, None, 702, w0, w_pre, base, scale, good, ws)
    torch.cuda.synchronize()
    ref, _ = oracle.decode_attention(_f64(qb)[:, 0], _f64(kb), _f64(vb), 702, w0, w_pre, base, scale)
    assert max_err(out.cpu().numpy()[:, 0], ref) <= TOL_BF16
