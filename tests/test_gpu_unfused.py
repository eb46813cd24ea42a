"""GPU parity of jl_bifocal_prefill_unfused: three separate attention passes
(A: stored view over each row's window, B: corrected view over all causal
keys, C: corrected view over the window) and their inclusion-exclusion merge
(Jet-Long §3.3 Eq. 6).  Compared with the oracle's literal three-pass merge,
with the dense bifocal definition it equals (pinned on the CPU), and with the
fused kernel."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, TOL_F32, assert_bf16_out_close, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _run(w, out_dtype, x=None):
    if x is None:
        x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    out = torch.empty((w.B, w.L, w.Hq, w.D), dtype=out_dtype, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_prefill_unfused(q, k, v, out, lse, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)
    torch.cuda.synchronize()
    return x, out, lse, (q, k, v, table)


CASES = [  # (B, L, Hq, Hkv, D, w_pre, w0)
    (1, 1000, 8, 2, 128, 300, 64),     # G = 4, window edge inside tiles, ragged end
    (2, 777, 4, 4, 64, 256, 100),      # G = 4, D = 64, no GQA
    (1, 1537, 16, 2, 128, 512, 200),   # G = 4, GQA 8
    (1, 600, 4, 2, 128, 256, 0),       # w0 = 0: only the diagonal in the window
    (1, 400, 4, 2, 128, 1000, 50),     # G = 1: the views coincide
    (1, 300, 4, 2, 128, 100, 400),     # w0 >= L: every pair in the window
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_L{c[1]}_H{c[2]}x{c[3]}_D{c[4]}_wp{c[5]}_w0{c[6]}"
                                              for c in CASES])
def test_unfused_matches_oracle(case):
    require_gpu()
    B, L, Hq, Hkv, D, w_pre, w0 = case
    w = si.Workload(f"unfused{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, 700 + L)
    x, o32, l32, _ = _run(w, torch.float32)
    _, o16, _, _ = _run(w, torch.bfloat16, x)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale)
    ie = oracle.inclusion_exclusion_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale)
    o32 = o32.cpu().numpy()
    print(case, "G", oracle.group_size(L, w_pre), "err", max_err(o32, ref), "vs IE", max_err(o32, ie),
          "lse", max_err(l32.cpu().numpy(), ref_lse))
    assert np.all(np.isfinite(o32))
    assert max_err(o32, ie) <= TOL_BF16
    assert max_err(o32, ref) <= TOL_BF16
    assert max_err(l32.cpu().numpy(), ref_lse) <= TOL_BF16
    assert_bf16_out_close(o16.float().cpu().numpy(), ref)


def test_unfused_fp32_matches_oracle_1e5():
    require_gpu()
    w = si.Workload("unfused_f32", "f32", 1, 512, 4, 2, 64, 64, 256, 1e4, 1001)
    x, out, lse, _ = _run(w, torch.float32)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w.w0, w.w_pretrained, w.rope_base,
                                            w.sm_scale)
    e, el = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    print("fp32 unfused err", e, "lse", el)
    assert e <= TOL_F32 and el <= TOL_F32


def test_unfused_agrees_with_fused():
    require_gpu()
    w = si.Workload("unfused_vs_fused", "bf16", 1, 2500, 32, 8, 128, 1024, 600, 1e6, 77)
    x, uo, ul, (q, k, v, table) = _run(w, torch.float32)
    fo, fl = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32, table)
    d, dl = max_err(uo.cpu().numpy(), fo.cpu().numpy()), max_err(ul.cpu().numpy(), fl.cpu().numpy())
    print("unfused vs fused", d, dl)
    # each side is within 2e-2 of the exact result; in practice they agree far closer
    assert d <= TOL_BF16 and dl <= TOL_BF16


# ---- the unfused decode step: three decode launches (A, B, C) and the merge
DEC_CASES = [  # (B, L, Lmax, Hq, Hkv, D, w_pre, w0)
    (1, 1500, 1600, 8, 2, 128, 400, 100),      # G = 4, window inside the cache
    (2, 777, 800, 4, 4, 64, 256, 33),          # G = 4, D = 64, no GQA, B = 2
    (1, 20000, 20000, 32, 8, 128, 4096, 1000), # many splits in every pass (two merge levels in B)
    (1, 600, 700, 8, 2, 128, 256, 0),          # w0 = 0: the window is the newest key
    (1, 400, 400, 8, 2, 128, 1000, 50),        # G = 1: the views coincide
    (1, 300, 310, 8, 2, 128, 100, 400),        # w0 >= L: the window holds every key
]


@pytest.mark.parametrize("case", DEC_CASES, ids=[f"B{c[0]}_L{c[1]}_H{c[3]}x{c[4]}_D{c[5]}_wp{c[6]}_w0{c[7]}"
                                                  for c in DEC_CASES])
def test_unfused_decode_matches_oracle(case):
    require_gpu()
    B, L, Lmax, Hq, Hkv, D, w_pre, w0 = case
    base, scale = 1e4, D ** -0.5
    rng = np.random.default_rng(L + 31 * Hq)
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    qb, kb, vb = bits((B, 1, Hq, D)), bits((B, Lmax, Hkv, D)), bits((B, Lmax, Hkv, D))
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_unfused_workspace(B, Hq, D, Lmax)
    fws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    f64 = lambda a: si.f32_from_bf16_bits(a).astype(np.float64)
    q64, k64, v64 = f64(qb)[:, 0], f64(kb), f64(vb)
    ref, ref_lse = oracle.decode_attention(q64, k64, v64, L, w0, w_pre, base, scale)
    # the oracle's literal three-softmax merge for the same row (query at L-1)
    qfull = np.zeros((B, L, Hq, D))
    qfull[:, L - 1] = q64
    ie = oracle.inclusion_exclusion_attention(qfull, k64[:, :L], v64[:, :L], w0, w_pre, base, scale,
                                              rows=np.array([L - 1]))[:, 0]
    outs = {}
    for od in (torch.float32, torch.bfloat16):
        out = torch.empty((B, 1, Hq, D), dtype=od, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        jl.jl_bifocal_decode_unfused(q, kc, vc, out, lse, L, w0, w_pre, base, scale, table, ws)
        torch.cuda.synchronize()
        outs[od] = (out.float().cpu().numpy()[:, 0], lse.cpu().numpy())
    fused = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode(q, kc, vc, fused, None, L, w0, w_pre, base, scale, table, fws)
    torch.cuda.synchronize()
    o32, l32 = outs[torch.float32]
    print(case, "G", oracle.group_size(L, w_pre), "unfused decode err", max_err(o32, ref), "vs IE",
          max_err(o32, ie), "lse", max_err(l32, ref_lse), "vs fused", max_err(o32, fused.cpu().numpy()[:, 0]))
    assert np.all(np.isfinite(o32))
    assert max_err(o32, ref) <= TOL_BF16 and max_err(o32, ie) <= TOL_BF16
    assert max_err(l32, ref_lse) <= TOL_BF16
    assert_bf16_out_close(outs[torch.bfloat16][0], ref, label=f"unfused decode {case}")
    assert max_err(o32, fused.cpu().numpy()[:, 0]) <= TOL_BF16
