"""GPU parity at one million tokens: a 256K-native model extended 4x
(Jet-Long §3.1 Eq. 2: G = ceil(1048576 / 262144) = 4), one KV head and its
four query heads.  This exercises the correction table over ~786K offsets,
64-bit offsets in every kernel, and decode steps on both sides of the G
transition at L = 2^20 (G = 4 at L = 2^20, G = 5 at L = 2^20 + 1).

The prefill runs in full on the GPU; the float64 oracle recomputes the
structural rows and 256 seeded rows.  Decode checks its rows one by one."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, oracle_rows_parallel, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(900)
def test_1m_prefill_sampled_rows_and_decode_across_g():
    require_gpu()
    w = si.WORKLOADS["ext1m"]
    assert oracle.group_size(w.L, w.w_pretrained) == 4
    print("[1m] generating inputs", flush=True)
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], w.dtype) for n in "qkv")
    Lmax = w.L + 2
    # sized for the pretrained window: offsets below n(Lmax - 1) + 1 under G(Lmax) = 5
    table = jl.alloc_table(Lmax, w.D, w.rope_base, w_pretrained=w.w_pretrained)
    print(f"[1m] correction table {table.numel()} bytes", flush=True)
    assert table.numel() < 1_100_000

    print("[1m] GPU prefill", flush=True)
    out, lse = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32, table)
    assert torch.isfinite(out).all()
    rows = si.sampled_rows(w.L, w.w0, w.w_pretrained, n_random=256, seed=w.seed)
    o_rows = out[:, rows].cpu().numpy()
    l_rows = lse[:, :, rows].cpu().numpy()
    del out, lse

    # the last 16 tokens as one chunk over the whole cache: 64 (position, query
    # head) columns on the decode kernels' staged path, 256 key splits
    print("[1m] 16-token chunk", flush=True)
    Lq = 16
    co = torch.empty((w.B, Lq, w.Hq, w.D), dtype=torch.float32, device="cuda")
    cl = torch.empty((w.B, w.Hq, Lq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_prefill_chunk(q[:, w.L - Lq:].contiguous(), k, v, co, cl, w.L, w.w0, w.w_pretrained, w.rope_base,
                                w.sm_scale, table)
    torch.cuda.synchronize()
    c_rows = np.arange(w.L - Lq, w.L)
    co, cl = co.cpu().numpy(), cl.cpu().numpy()
    del q

    print(f"[1m] oracle on {len(rows)} rows x {w.Hq} heads", flush=True)
    q64 = np.zeros((w.B, w.L, w.Hq, w.D))
    q64[:, rows] = si.f32_from_bf16_bits(x["q"][:, rows])
    k64 = si.f32_from_bf16_bits(x["k"]).astype(np.float64)
    v64 = si.f32_from_bf16_bits(x["v"]).astype(np.float64)
    ref, ref_lse = oracle_rows_parallel(q64, k64, v64, rows, w.w0, w.w_pretrained, w.rope_base, w.sm_scale,
                                        workers=8)
    del q64
    e, el = max_err(o_rows, ref), max_err(l_rows, ref_lse)
    print(f"[1m] prefill err {e:.3e}, lse err {el:.3e}", flush=True)
    assert e <= TOL_BF16 and el <= TOL_BF16

    q64 = np.zeros((w.B, w.L, w.Hq, w.D))
    q64[:, c_rows] = si.f32_from_bf16_bits(x["q"][:, c_rows])
    cref, cref_lse = oracle_rows_parallel(q64, k64, v64, c_rows, w.w0, w.w_pretrained, w.rope_base, w.sm_scale,
                                          workers=8)
    del q64
    ce, cel = max_err(co, cref), max_err(cl, cref_lse)
    print(f"[1m] 16-token chunk err {ce:.3e}, lse err {cel:.3e}", flush=True)
    assert ce <= TOL_BF16 and cel <= TOL_BF16

    # two decode steps: a query at position 2^20 - 1 over the prefilled cache
    # (L = 2^20, G = 4), then one more key appended (L = 2^20 + 1, G = 5)
    kc = torch.zeros((w.B, Lmax, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kc[:, :w.L] = k
    vc[:, :w.L] = v
    del k, v
    ws = jl.alloc_decode_workspace(w.B, w.Hq, w.D, Lmax)
    rng = np.random.Generator(np.random.PCG64([w.seed, 11]))
    kfull, vfull = k64, v64
    for L in (w.L, w.L + 1):
        G = oracle.group_size(L, w.w_pretrained)
        qb = si.bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hq, w.D), dtype=np.float32))
        if L > w.L:
            kb = si.bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hkv, w.D), dtype=np.float32))
            vb = si.bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hkv, w.D), dtype=np.float32))
            kc[:, L - 1:L] = to_dev(kb, "bf16")
            vc[:, L - 1:L] = to_dev(vb, "bf16")
            kfull = np.concatenate([kfull, si.f32_from_bf16_bits(kb).astype(np.float64)], axis=1)
            vfull = np.concatenate([vfull, si.f32_from_bf16_bits(vb).astype(np.float64)], axis=1)
        dout = torch.empty((w.B, 1, w.Hq, w.D), dtype=torch.float32, device="cuda")
        dlse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        jl.jl_bifocal_decode(to_dev(qb, "bf16"), kc, vc, dout, dlse, L, w.w0, w.w_pretrained, w.rope_base,
                             w.sm_scale, table, ws)
        torch.cuda.synchronize()
        q_tok = si.f32_from_bf16_bits(qb)[:, 0].astype(np.float64)
        dref, dref_lse = oracle.decode_attention(q_tok, kfull[:, :L], vfull[:, :L], L, w.w0, w.w_pretrained,
                                                 w.rope_base, w.sm_scale)
        de, dle = max_err(dout.cpu().numpy()[:, 0], dref), max_err(dlse.cpu().numpy(), dref_lse)
        print(f"[1m] decode L={L} (G={G}) err {de:.3e}, lse err {dle:.3e}", flush=True)
        assert de <= TOL_BF16 and dle <= TOL_BF16
