"""GPU check of jl_bifocal_decode_noalloc (the decode step for callers that
cannot allocate: its split partials live in the library's fixed device
scratch): called through the C ABI, it must give what jl_bifocal_decode gives
with a workspace, to the parity bar (here bit for bit: the same kernels and
plan), on two calls in a row, the second with a smaller input (the scratch
keeps the first call's contents), and both within 2e-2 of the oracle.  Also:
a step whose partials exceed the fixed scratch is refused before any HIP
call, leaving the output untouched."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _case(B, L, Lmax, Hq, Hkv, D, w_pre, w0, seed, out_dtype):
    base, scale = 1e6, D ** -0.5
    rng = np.random.default_rng(seed)
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    qb, kb, vb = bits((B, 1, Hq, D)), bits((B, Lmax, Hkv, D)), bits((B, Lmax, Hkv, D))
    q, kc, vc = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
    table = jl.alloc_table(Lmax, D, base)
    ws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    ref_out = torch.empty((B, 1, Hq, D), dtype=out_dtype, device="cuda")
    ref_lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode(q, kc, vc, ref_out, ref_lse, L, w0, w_pre, base, scale, table, ws)
    torch.cuda.synchronize()
    f64 = lambda a: si.f32_from_bf16_bits(a).astype(np.float64)
    exact, exact_lse = oracle.decode_attention(f64(qb)[:, 0], f64(kb), f64(vb), L, w0, w_pre, base, scale)
    return (q, kc, vc, table, base, scale), ref_out, ref_lse, exact, exact_lse


def _noalloc(args, L, w0, w_pre, out_dtype):
    q, kc, vc, table, base, scale = args
    B, _, Hq, D = q.shape
    out = torch.full((B, 1, Hq, D), float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    rc = jl.lib.jl_bifocal_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(vc.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()), jl.JL_BF16,
        jl.JL_BF16 if out_dtype == torch.bfloat16 else jl.JL_F32, B, L, kc.shape[1], Hq, kc.shape[2], D, w0, w_pre,
        base, scale, ctypes.c_void_p(table.data_ptr()), table.numel(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == jl.JL_OK, jl.jl_last_error()
    torch.cuda.synchronize()
    return out, lse


def test_noalloc_decode_equals_workspace_decode_twice():
    require_gpu()
    # first: the 128K-cache shape (128 splits per KV-head group, 2 MiB of partials)
    big = dict(B=1, L=131073, Lmax=131200, Hq=32, Hkv=8, D=128, w_pre=32768, w0=4096)
    # second, smaller: fewer heads, a shorter cache, two sequences
    small = dict(B=2, L=1500, Lmax=1600, Hq=8, Hkv=2, D=128, w_pre=400, w0=100)
    for i, (c, od) in enumerate(((big, torch.bfloat16), (small, torch.float32))):
        args, ref_out, ref_lse, exact, exact_lse = _case(c["B"], c["L"], c["Lmax"], c["Hq"], c["Hkv"], c["D"],
                                                         c["w_pre"], c["w0"], 50 + i, od)
        out, lse = _noalloc(args, c["L"], c["w0"], c["w_pre"], od)
        print(f"[no-alloc] call {i + 1}: L={c['L']} B={c['B']} Hq={c['Hq']}: equal to the workspace call: "
              f"{torch.equal(out, ref_out) and torch.equal(lse, ref_lse)}, vs oracle "
              f"{max_err(out.float().cpu().numpy()[:, 0], exact):.3e}", flush=True)
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        assert max_err(out.float().cpu().numpy()[:, 0], exact) <= TOL_BF16
        assert max_err(lse.cpu().numpy(), exact_lse) <= TOL_BF16


def test_noalloc_refuses_a_step_beyond_its_scratch():
    require_gpu()
    # B * Hq * n_split * (D + 2) * 4 bytes: 1024 sequences of 64 query heads over 8 KV heads fill
    # 2048 workgroups, so each head has one split -> 1024 * 64 * 130 * 4 = 32.5 MiB > 16 MiB.
    # Validation fails before any HIP call, so the buffers below are never read (tiny stand-ins
    # of the right alignment).
    t = torch.zeros(1024, dtype=torch.bfloat16, device="cuda")
    out = torch.full((16,), 7.0, device="cuda")
    tab = jl.alloc_table(8, 128, 1e6)
    rc = jl.lib.jl_bifocal_decode_noalloc(
        ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(t.data_ptr()), ctypes.c_void_p(t.data_ptr()),
        ctypes.c_void_p(out.data_ptr()), None, jl.JL_BF16, jl.JL_F32, 1024, 64, 64, 64, 8, 128, 16, 32,
        1e6, 0.088, ctypes.c_void_p(tab.data_ptr()), 1 << 40, None)
    torch.cuda.synchronize()
    assert rc == jl.JL_ESPACE and "scratch" in jl.jl_last_error()
    assert bool((out == 7.0).all())
