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
from gpu_common import (TOL_BF16, TOL_F32, assert_bf16_out_close, max_err, oracle_rows_parallel, prefill,
                        require_gpu, to_dev)

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


def test_unsplit_chunk_equals_full_prefill_rows():
    """Below 8 key tiles a chunk on the prefill kernels is not split: it walks every
    row's key tiles in the order of the full prefill, so the two agree bit for bit.
    (Chunks of at most 64 columns, here 16 tokens, run on the decode kernels and are
    checked against the oracle below.)"""
    require_gpu()
    w = _workload(896, 8, 2, 128, 256, 100, seed=9)
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    full, lse_full = prefill(q, k, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32, table)
    for Lq in (17, 64, 333, 896):
        _, out, lse = _run_chunk(w, Lq, w.L, torch.float32, x)
        d = max_err(out.cpu().numpy(), full[:, w.L - Lq:].cpu().numpy())
        dl = max_err(lse.cpu().numpy(), lse_full[:, :, w.L - Lq:].cpu().numpy())
        print("Lq", Lq, "chunk vs full", d, dl)
        assert d == 0 and dl == 0


def test_split_chunk_agrees_with_full_prefill_rows():
    """Short chunks over 16 key tiles are split over workgroups and merged by
    log-sum-exp (on the prefill kernels, or for one token on the decode kernels):
    the same rows as the full prefill up to rounding."""
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
        print("Lq", Lq, "split chunk vs full", d, dl)
        assert d <= 5e-3 and dl <= 5e-3


def test_chunk_state_rotates_only_new_keys():
    """A sequence prefilled chunk by chunk with one workspace and its state:
    each chunk rotates only the key rows the state lacks (and all of them
    when G changes; a short chunk on the decode kernels none, when the state
    covers the rows it reads rotated), and every chunk equals the stateless
    call bit for bit."""
    require_gpu()
    w = _workload(1400, 8, 2, 128, 400, 100, seed=44)   # G = 1 up to 400, 2 to 800, 3 to 1200, then 4
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    Lmax = 1500
    kc = torch.zeros((1, Lmax, w.Hkv, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    table = jl.alloc_table(Lmax, w.D, w.rope_base)
    st = jl.alloc_chunk_state(q[:, :300], kc, w.w_pretrained)
    L = 0
    for Lq in (300, 200, 1, 256, 43, 300, 300):   # crosses 400, 800 and 1200
        L += Lq
        kc[:, L - Lq:L], vc[:, L - Lq:L] = k[:, L - Lq:L], v[:, L - Lq:L]
        qc = q[:, L - Lq:L].contiguous()
        a = torch.empty((1, Lq, w.Hq, w.D), dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        G = oracle.group_size(L, w.w_pretrained)
        before = (st.state.G, st.state.rows)
        jl.jl_bifocal_prefill_chunk(qc, kc, vc, a, None, L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table,
                                    workspace=st)
        jl.jl_bifocal_prefill_chunk(qc, kc, vc, b, None, L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)
        torch.cuda.synchronize()
        print(f"L={L} Lq={Lq} G={G} state {before} -> {(st.state.G, st.state.rows)}")
        on_decode = Lq * (w.Hq // w.Hkv) <= 64
        if G > 1 and on_decode and before[0] == G and L - 1 - w.w0 <= before[1] <= L:
            # on the decode kernels, rows below L-1-w0 are all the chunk reads
            # rotated: a state that covers them is left as it is
            assert (st.state.G, st.state.rows) == before
        else:
            assert (st.state.G, st.state.rows) == (G, L if G > 1 else 0)
        assert torch.equal(a, b)


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


@pytest.mark.timeout(600)
def test_short_chunks_at_128k_match_oracle():
    """Chunks of 1, 16 and 256 tokens at the end of the 128K workload (G = 4),
    in the configuration the benchmark times (1 and 16 tokens on the decode
    kernels, 256 on the split prefill kernels), against the oracle on every
    chunk row (up to 64 seeded rows of the 256-token chunk), all heads."""
    require_gpu()
    w = si.WORKLOADS["ext128k"]
    x = si.make_prefill_inputs(w, want_f64=False)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base, w_pretrained=w.w_pretrained)
    k64 = si.f32_from_bf16_bits(x["k"]).astype(np.float64)
    v64 = si.f32_from_bf16_bits(x["v"]).astype(np.float64)
    rng = np.random.default_rng(5)
    for Lq in (1, 16, 256):
        qc = q[:, w.L - Lq:].contiguous()
        out = torch.empty((w.B, Lq, w.Hq, w.D), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.Hq, Lq), dtype=torch.float32, device="cuda")
        jl.jl_bifocal_prefill_chunk(qc, k, v, out, lse, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)
        torch.cuda.synchronize()
        idx = np.arange(Lq) if Lq <= 64 else np.sort(rng.choice(Lq, 64, replace=False))
        rows = w.L - Lq + idx
        q64 = np.zeros((w.B, w.L, w.Hq, w.D))
        q64[:, rows] = si.f32_from_bf16_bits(x["q"][:, rows])
        ref, ref_lse = oracle_rows_parallel(q64, k64, v64, rows, w.w0, w.w_pretrained, w.rope_base, w.sm_scale)
        e = max_err(out.cpu().numpy()[:, idx], ref)
        el = max_err(lse.cpu().numpy()[:, :, idx], ref_lse)
        print(f"[chunk128k] Lq={Lq}: {len(idx)} rows x {w.Hq} heads, err {e:.3e}, lse err {el:.3e}", flush=True)
        assert e <= TOL_BF16 and el <= TOL_BF16


SHORT = [  # (B, L, Lq, Hq, Hkv, D, w_pre, w0): chunks of at most 64 columns per KV head
    (1, 3000, 1, 32, 8, 128, 700, 300),    # one token, 4 of 16 columns, G = 5
    (2, 2500, 3, 8, 2, 128, 600, 100),     # 12 columns, two sequences
    (1, 2000, 7, 8, 2, 128, 512, 5),       # two groups (28 columns); w0 < Lq: the window edges differ per column
    (1, 4100, 16, 32, 8, 128, 1024, 40),   # four groups of 16, the benchmark's shape on a shorter cache
    (1, 1500, 13, 8, 2, 64, 400, 9),       # D = 64, 52 of 64 columns
    (1, 20, 16, 4, 4, 128, 8, 2),          # the chunk is the whole sequence: early columns see few keys
    (1, 900, 64, 8, 8, 128, 300, 50),      # GQA 1: 64 positions in four groups
    (1, 1000, 8, 16, 2, 128, 256, 100),    # GQA 8: 64 columns
    (1, 600, 10, 8, 2, 128, 4096, 50),     # G = 1
    (1, 300, 16, 8, 2, 64, 1, 3),          # w_pre = 1: G = L, every remote key at position 0
    (1, 500, 12, 8, 2, 128, 256, 600),     # w0 >= L: every key local although G = 2
]


@pytest.mark.parametrize("case", SHORT, ids=[f"B{c[0]}_L{c[1]}_Lq{c[2]}_H{c[3]}x{c[4]}_D{c[5]}" for c in SHORT])
def test_short_chunk_on_decode_kernels_matches_oracle(case):
    """Short chunks run as decode steps with several query positions (one MFMA
    column per (position, query head)): every row against the oracle, fp32 and
    bf16 outputs, and the same call over a shuffled paged copy of the cache
    bit for bit."""
    require_gpu()
    B, L, Lq, Hq, Hkv, D, w_pre, w0 = case
    w = si.Workload(f"short{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, L + 7 * Lq)
    x, o32, l32 = _run_chunk(w, Lq, L + 40, torch.float32)
    _, o16, _ = _run_chunk(w, Lq, L + 40, torch.bfloat16, x)
    rows = np.arange(L - Lq, L)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w0, w_pre, w.rope_base, w.sm_scale,
                                            rows=rows)
    o32 = o32.cpu().numpy()
    e, el = max_err(o32, ref), max_err(l32.cpu().numpy(), ref_lse)
    print(f"[short chunk] {case} G {oracle.group_size(L, w_pre)}: err {e:.3e}, lse err {el:.3e}", flush=True)
    assert np.all(np.isfinite(o32))
    assert e <= TOL_BF16 and el <= TOL_BF16
    assert_bf16_out_close(o16.float().cpu().numpy(), ref)
    # the paged form: pages of 128 keys in a shuffled order
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    ps = 128
    n_p = -(-L // ps)
    perm = torch.randperm(B * n_p, generator=torch.Generator().manual_seed(L)).to(torch.int32)
    kp = torch.zeros((B * n_p, ps, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    bt = perm.view(B, n_p).cuda()
    for bb in range(B):
        for j in range(n_p):
            n = min(ps, L - j * ps)
            kp[perm[bb * n_p + j], :n] = k[bb, j * ps:j * ps + n]
            vp[perm[bb * n_p + j], :n] = v[bb, j * ps:j * ps + n]
    out = torch.empty((B, Lq, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq, Lq), dtype=torch.float32, device="cuda")
    table = jl.alloc_table(L, D, w.rope_base)
    jl.jl_bifocal_prefill_chunk_paged(q[:, L - Lq:].contiguous(), kp, vp, bt, out, lse, L, w0, w_pre, w.rope_base,
                                      w.sm_scale, table)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), o32) and np.array_equal(lse.cpu().numpy(), l32.cpu().numpy())
