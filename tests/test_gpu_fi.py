"""GPU parity of the frequency-interpolation remote view (Jet-Long §4.7
ablation; s = max(1, L / w_pretrained) from §3.1): jl_bifocal_prefill_fi and
jl_bifocal_decode_fi against the float64 oracle (its view pinned on the CPU
by a brute force from raw vectors), the s = 1 reduction to the plain path,
and a table built for another call."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, TOL_F32, assert_bf16_out_close, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _prefill_fi(w, x, out_dtype, alpha, beta, table=None):
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    if table is None:
        table = jl.alloc_fi_table(w.L, w.w_pretrained, w.D, w.rope_base, alpha, beta)
    out = torch.empty((w.B, w.L, w.Hq, w.D), dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_prefill_fi(q, k, v, out, lse, w.w0, w.w_pretrained, w.rope_base, alpha, beta, w.sm_scale, table)
    torch.cuda.synchronize()
    return out, lse, (q, k, v)


CASES = [  # (B, L, Hq, Hkv, D, w_pre, w0, alpha, beta)
    (1, 1000, 8, 2, 128, 300, 64, 1.0, 32.0),      # s = 3.33, YaRN's bounds
    (2, 777, 4, 4, 64, 256, 100, 1.0, 32.0),       # D = 64, no GQA
    (1, 1537, 16, 2, 128, 512, 200, 0.5, 8.0),     # GQA 8
    (1, 600, 4, 2, 128, 256, 0, 50.0, 100.0),      # every pair divided by s (position interpolation)
    (1, 900, 8, 2, 128, 100, 30, -2.0, -1.0),      # every pair kept: plain attention
    (1, 300, 16, 2, 128, 100, 400, 1.0, 32.0),     # w0 >= L: every pair local, s = 3
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_L{c[1]}_H{c[2]}x{c[3]}_D{c[4]}_wp{c[5]}_w0{c[6]}_a{c[7]}"
                                              for c in CASES])
def test_prefill_fi_matches_oracle(case):
    require_gpu()
    B, L, Hq, Hkv, D, w_pre, w0, alpha, beta = case
    w = si.Workload(f"fi{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, 900 + L)
    x = si.make_prefill_inputs(w)
    o32, l32, _ = _prefill_fi(w, x, torch.float32, alpha, beta)
    o16, _, _ = _prefill_fi(w, x, torch.bfloat16, alpha, beta)
    ref, ref_lse = oracle.bifocal_attention_fi(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, alpha, beta,
                                               w.sm_scale)
    o32 = o32.cpu().numpy()
    e, el = max_err(o32, ref), max_err(l32.cpu().numpy(), ref_lse)
    print(case, "s", oracle.fi_scale(L, w_pre), "err", e, "lse", el)
    assert np.all(np.isfinite(o32))
    assert e <= TOL_BF16 and el <= TOL_BF16
    assert_bf16_out_close(o16.float().cpu().numpy(), ref)


def test_prefill_fi_fp32_matches_oracle_1e5():
    require_gpu()
    w = si.Workload("fi_f32", "f32", 1, 512, 4, 2, 64, 64, 200, 1e4, 1001)
    x = si.make_prefill_inputs(w)
    out, lse, _ = _prefill_fi(w, x, torch.float32, 1.0, 32.0)
    ref, ref_lse = oracle.bifocal_attention_fi(x["q64"], x["k64"], x["v64"], w.w0, w.w_pretrained, w.rope_base,
                                               1.0, 32.0, w.sm_scale)
    e, el = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    print("fp32 fi err", e, "lse", el)
    assert e <= TOL_F32 and el <= TOL_F32


def test_prefill_fi_within_the_window_is_the_plain_path():
    """L <= w_pretrained: s = 1 and G = 1, both calls are the same plain
    attention, bit for bit."""
    require_gpu()
    w = si.Workload("fi_s1", "bf16", 1, 700, 8, 2, 128, 50, 700, 1e4, 5)
    x = si.make_prefill_inputs(w)
    o, l, (q, k, v) = _prefill_fi(w, x, torch.float32, 1.0, 32.0)
    po, pl = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32,
                     jl.alloc_table(w.L, w.D, w.rope_base))
    torch.cuda.synchronize()
    assert torch.equal(o, po) and torch.equal(l, pl)


def test_prefill_fi_refuses_a_table_for_another_call():
    """The kernels compare the table header with the call: an offset table, or
    an interpolation table for another L or ramp, gives NaN outputs."""
    require_gpu()
    w = si.Workload("fi_bad", "bf16", 1, 600, 8, 2, 128, 30, 200, 1e4, 6)
    x = si.make_prefill_inputs(w)
    for bad in (jl.alloc_table(w.L, w.D, w.rope_base),
                jl.alloc_fi_table(w.L + 1, w.w_pretrained, w.D, w.rope_base, 1.0, 32.0),
                jl.alloc_fi_table(w.L, w.w_pretrained, w.D, w.rope_base, 1.0, 16.0)):
        o, l, _ = _prefill_fi(w, x, torch.float32, 1.0, 32.0, table=bad)
        assert torch.isnan(o).all() and torch.isnan(l).all()


def _cache(B, Lmax, Hq, Hkv, D, seed):
    rng = np.random.Generator(np.random.PCG64([seed, 21]))
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    return bits((B, 1, Hq, D)), bits((B, Lmax, Hkv, D)), bits((B, Lmax, Hkv, D))


def _f64(a):
    return si.f32_from_bf16_bits(a).astype(np.float64)


DCASES = [  # (B, L, Lmax, Hq, Hkv, D, w_pre, w0, alpha, beta)
    (2, 1537, 1600, 8, 2, 128, 400, 100, 1.0, 32.0),
    (1, 1000, 1100, 4, 2, 64, 300, 64, 1.0, 32.0),
    (1, 20000, 20050, 32, 8, 128, 4096, 1000, 1.0, 32.0),   # many splits, s = 4.88
    (1, 600, 700, 8, 8, 128, 256, 0, 50.0, 100.0),
    (1, 131328, 131328, 32, 8, 128, 32768, 4096, 1.0, 32.0),  # the 128K cache, angles up to ~1e5 rad
    (2, 300, 320, 16, 2, 128, 100, 400, 1.0, 32.0),          # w0 >= L: no remote key
    (1, 65, 70, 4, 2, 64, 1, 3, 1.0, 32.0),                  # w_pretrained = 1: s = L
]


@pytest.mark.parametrize("case", DCASES, ids=[f"B{c[0]}_L{c[1]}_H{c[3]}x{c[4]}_D{c[5]}_wp{c[6]}_w0{c[7]}"
                                                for c in DCASES])
def test_decode_fi_matches_oracle(case):
    require_gpu()
    B, L, Lmax, Hq, Hkv, D, w_pre, w0, alpha, beta = case
    base, scale = 1e6 if L > 100000 else 1e4, D ** -0.5
    qb, kb, vb = _cache(B, Lmax, Hq, Hkv, D, seed=L + Hq)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode_fi(q, kc, vc, out, lse, L, w0, w_pre, base, alpha, beta, scale, ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_attention_fi(_f64(qb)[:, 0], _f64(kb), _f64(vb), L, w0, w_pre, base, alpha, beta,
                                              scale)
    e, el = max_err(out.cpu().numpy()[:, 0], ref), max_err(lse.cpu().numpy(), ref_lse)
    print(case, "s", oracle.fi_scale(L, w_pre), "err", e, "lse", el)
    assert e <= TOL_BF16 and el <= TOL_BF16


def test_decode_fi_steps_and_s1():
    """Consecutive steps (s changes with every L) against the oracle, and a
    step with L <= w_pretrained equal to the plain decode bit for bit."""
    require_gpu()
    B, Lmax, Hq, Hkv, D, w_pre, w0, base = 1, 1200, 8, 2, 128, 400, 50, 1e4
    scale = D ** -0.5
    qb, kb, vb = _cache(B, Lmax, Hq, Hkv, D, seed=8)
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    out = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    for L in (1100, 1101, 1102, 1199):
        jl.jl_bifocal_decode_fi(q, kc, vc, out, None, L, w0, w_pre, base, 1.0, 32.0, scale, ws)
        torch.cuda.synchronize()
        ref, _ = oracle.decode_attention_fi(_f64(qb)[:, 0], _f64(kb), _f64(vb), L, w0, w_pre, base, 1.0, 32.0, scale)
        e = max_err(out.cpu().numpy()[:, 0], ref)
        print("L", L, "err", e)
        assert e <= TOL_BF16
    plain = torch.empty_like(out)
    jl.jl_bifocal_decode_fi(q, kc, vc, out, None, 390, w0, w_pre, base, 1.0, 32.0, scale, ws)
    jl.jl_bifocal_decode(q, kc, vc, plain, None, 390, w0, w_pre, base, scale, jl.alloc_table(Lmax, D, base), ws)
    torch.cuda.synchronize()
    assert torch.equal(out, plain)


def test_device_fi_table_equals_host_fi_table():
    """The device fill and the host fill of the interpolation table agree:
    header bit for bit, entries within one fp32 ulp (device and host float64
    cos/sin may round differently)."""
    require_gpu()
    for (L, w_pre, D, base, alpha, beta) in [(1000, 300, 64, 1e4, 1.0, 32.0),
                                             (131328, 32768, 128, 1e6, 1.0, 32.0)]:
        t = jl.alloc_fi_table(L, w_pre, D, base, alpha, beta)
        torch.cuda.synchronize()
        dev = t.cpu().numpy()
        host = jl.jl_fi_table_fill_host(L, w_pre, D, base, alpha, beta)
        assert np.array_equal(dev[:64], host[:64])
        a = dev[64:].view(np.float32).astype(np.float64)
        b = host[64:].view(np.float32)
        assert np.all(np.abs(a - b) <= np.spacing(np.abs(b)).astype(np.float64) + 1e-10)
