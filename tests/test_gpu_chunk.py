"""GPU parity of jl_bifocal_prefill_chunk: Lq new tokens at positions
L-Lq .. L-1 over a cache of L keys are the last Lq rows of the prefill over
L tokens, under G(L) (Jet-Long §3.1 Eq. 2 with §3.2 Eqs. 4-5).  The oracle is
the float64 prefill definition restricted to those rows."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, TOL_F32, assert_bf16_out_close, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _workload(L, Hq, Hkv, D, w_pre, w0, dtype="bf16", B=1, seed=31):
    return si.Workload(f"chunk{L}", dtype, B, L, Hq, Hkv, D, w0, w_pre, 1e4, seed)


def _run_chunk(w, Lq, Lmax, out_dtype, x=None):
    """The chunk call on caches of Lmax rows whose rows >= L hold NaN."""
    if x is None:
        x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    dt = q.dtype
    kc = torch.full((w.B, Lmax, w.Hkv, w.D), float("nan"), dtype=dt, device=q.device)
    vc = torch.full_like(kc, float("nan"))
    kc[:, :w.L] = k
    vc[:, :w.L] = v
    qc = q[:, w.L - Lq:].contiguous()
    out = torch.empty((w.B, Lq, w.Hq, w.D), dtype=out_dtype, device=q.device)
    lse = torch.empty((w.B, w.Hq, Lq), dtype=torch.float32, device=q.device)
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    jl.jl_bifocal_prefill_chunk(qc, kc, vc, out, lse, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)
    torch.cuda.synchronize()
    return x, out, lse


CASES = [  # (L, Lq, Lmax, Hq, Hkv, D, w_pre, w0)
    (1000, 300, 1100, 8, 2, 128, 300, 64),    # G = 4, offset 700 not tile aligned
    (612, 100, 612, 4, 2, 128, 256, 50),      # crosses 512 = 2 * w_pre: chunk under G = 3
    (777, 1, 800, 8, 2, 64, 256, 100),        # one token, D = 64
    (1537, 517, 1600, 16, 2, 128, 512, 200),  # GQA 8, ragged
    (300, 300, 300, 4, 4, 64, 1000, 30),      # the whole sequence, G = 1
]


@pytest.mark.parametrize("case", CASES, ids=[f"L{c[0]}_Lq{c[1]}_Lmax{c[2]}_H{c[3]}x{c[4]}_D{c[5]}" for c in CASES])
def test_chunk_matches_oracle_rows(case):
    require_gpu()
    L, Lq, Lmax, Hq, Hkv, D, w_pre, w0 = case
    w = _workload(L, Hq, Hkv, D, w_pre, w0, seed=L + Lq)
    x, o32, l32 = _run_chunk(w, Lq, Lmax, torch.float32)
    _, o16, _ = _run_chunk(w, Lq, Lmax, torch.bfloat16, x)
    rows = np.arange(L - Lq, L)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale,
                                            rows=rows)
    o32 = o32.cpu().numpy()
    print(case, "G", oracle.group_size(L, w_pre), "err", max_err(o32, ref), "lse", max_err(l32.cpu().numpy(), ref_lse))
    assert np.all(np.isfinite(o32))
    assert max_err(o32, ref) <= TOL_BF16
    assert max_err(l32.cpu().numpy(), ref_lse) <= TOL_BF16
    assert_bf16_out_close(o16.float().cpu().numpy(), ref)


def test_chunk_fp32_matches_oracle_1e5():
    require_gpu()
    w = _workload(700, 4, 2, 64, 200, 50, dtype="f32", seed=5)
    x, out, lse = _run_chunk(w, 250, 760, torch.float32)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w.w0, w.w_pretrained, w.rope_base,
                                            w.sm_scale, rows=np.arange(450, 700))
    assert max_err(out.cpu().numpy(), ref) <= TOL_F32
    assert max_err(lse.cpu().numpy(), ref_lse) <= TOL_F32


def test_chunk_equals_full_prefill_rows():
    """The chunk and the full prefill walk every row's key tiles in the same order, so their
    results agree bit for bit."""
    require_gpu()
    w = _workload(2000, 8, 2, 128, 512, 256, seed=9)
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    full, lse_full = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32, table)
    for Lq in (1, 64, 333, 2000):
        _, out, lse = _run_chunk(w, Lq, w.L, torch.float32, x)
        d = max_err(out.cpu().numpy(), full[:, w.L - Lq:].cpu().numpy())
        dl = max_err(lse.cpu().numpy(), lse_full[:, :, w.L - Lq:].cpu().numpy())
        print("Lq", Lq, "chunk vs full", d, dl)
        assert d == 0 and dl == 0


def test_one_token_chunk_equals_decode():
    require_gpu()
    w = _workload(1500, 8, 2, 128, 400, 128, seed=21)
    x, out, lse = _run_chunk(w, 1, 1600, torch.float32)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    ws = jl.alloc_decode_workspace(1, w.Hq, w.D, w.L)
    dout = torch.empty((1, 1, w.Hq, w.D), dtype=torch.float32, device="cuda")
    dlse = torch.empty((1, w.Hq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode(q[:, -1:].contiguous(), k, v, dout, dlse, w.L, w.w0, w.w_pretrained, w.rope_base,
                         w.sm_scale, table, ws)
    torch.cuda.synchronize()
    assert max_err(out.cpu().numpy(), dout.cpu().numpy()) <= 5e-3
    assert max_err(lse[:, :, 0].cpu().numpy(), dlse.cpu().numpy()) <= 5e-3
