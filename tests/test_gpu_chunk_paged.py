"""GPU parity of jl_bifocal_prefill_chunk_paged: a chunk of Lq tokens over a
cache held in shuffled pages equals the same chunk over the contiguous cache
bit for bit (Jet-Long §3 Eq. 1, §3.2 Eqs. 4-5: the keys are read as stored
wherever they sit), and the float64 oracle's rows.  A block-table entry
outside the pages is never followed: the rows that need it come out NaN."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _paginate(kc, vc, L, page_size, seed, spare=2):
    """The first L rows of each sequence in shuffled pages (plus unused
    pages filled with NaN) and the block table."""
    B, _, Hkv, D = kc.shape
    max_pages = (L + page_size - 1) // page_size
    n_pages = B * max_pages + spare
    perm = np.random.Generator(np.random.PCG64([seed, 9])).permutation(n_pages)[: B * max_pages]
    kp = torch.full((n_pages, page_size, Hkv, D), float("nan"), dtype=kc.dtype, device=kc.device)
    vp = torch.full_like(kp, float("nan"))
    for b in range(B):
        for s in range(max_pages):
            pg = int(perm[b * max_pages + s])
            n = min(page_size, L - s * page_size)
            kp[pg, :n] = kc[b, s * page_size:s * page_size + n]
            vp[pg, :n] = vc[b, s * page_size:s * page_size + n]
    bt = torch.from_numpy(perm.reshape(B, max_pages).astype(np.int32)).to(kc.device)
    return kp, vp, bt


def _setup(B, L, Lq, Hq, Hkv, D, w_pre, w0, seed):
    w = si.Workload(f"chunkpaged{L}", "bf16", B, L, Hq, Hkv, D, w0, w_pre, 1e4, seed)
    x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")
    qc = q[:, L - Lq:].contiguous()
    table = jl.alloc_table(L, D, w.rope_base)
    return w, x, qc, k, v, table


def _contig(w, qc, k, v, table, Lq):
    out = torch.empty((w.B, Lq, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, Lq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_prefill_chunk(qc, k, v, out, lse, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)
    return out, lse


def _paged(w, qc, kp, vp, bt, table, Lq):
    out = torch.empty((w.B, Lq, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, Lq), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_prefill_chunk_paged(qc, kp, vp, bt, out, lse, w.L, w.w0, w.w_pretrained, w.rope_base,
                                      w.sm_scale, table)
    return out, lse


CASES = [  # (B, L, Lq, Hq, Hkv, D, page_size, w_pre, w0)
    (2, 1000, 300, 8, 2, 128, 128, 300, 64),     # G = 4, offset 700 not tile aligned
    (1, 1537, 1537, 16, 2, 128, 256, 512, 200),  # the whole sequence as one chunk, GQA 8
    (1, 777, 1, 8, 2, 64, 128, 256, 100),        # one token, D = 64
    (1, 612, 100, 4, 2, 128, 512, 256, 50),      # crosses 2 * w_pre: under G = 3, one page for all
    (1, 300, 300, 4, 4, 64, 128, 1000, 30),      # G = 1: no rotated keys
]


@pytest.mark.parametrize("case", CASES, ids=[f"B{c[0]}_L{c[1]}_Lq{c[2]}_H{c[3]}x{c[4]}_D{c[5]}_ps{c[6]}"
                                              for c in CASES])
def test_chunk_paged_equals_contiguous(case):
    require_gpu()
    B, L, Lq, Hq, Hkv, D, ps, w_pre, w0 = case
    w, x, qc, k, v, table = _setup(B, L, Lq, Hq, Hkv, D, w_pre, w0, seed=L + Lq + ps)
    ref_o, ref_l = _contig(w, qc, k, v, table, Lq)
    kp, vp, bt = _paginate(k, v, L, ps, seed=L + ps)
    out, lse = _paged(w, qc, kp, vp, bt, table, Lq)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)


def test_chunk_paged_matches_oracle():
    require_gpu()
    w, x, qc, k, v, table = _setup(1, 1100, 400, 8, 2, 128, 350, 100, seed=4)
    kp, vp, bt = _paginate(k, v, w.L, 256, seed=5)
    out, lse = _paged(w, qc, kp, vp, bt, table, 400)
    torch.cuda.synchronize()
    rows = np.arange(w.L - 400, w.L)
    ref, ref_lse = oracle.bifocal_attention(x["q64"], x["k64"], x["v64"], w.w0, w.w_pretrained, w.rope_base,
                                            w.sm_scale, rows=rows)
    e, el = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    print("paged chunk err", e, "lse", el, "G", oracle.group_size(w.L, w.w_pretrained))
    assert e <= TOL_BF16 and el <= TOL_BF16


def test_out_of_range_page_poisons_the_rows_that_need_it():
    require_gpu()
    B, L, Lq, Hq, Hkv, D, ps, w_pre, w0 = 2, 1000, 600, 8, 2, 128, 128, 300, 64
    w, x, qc, k, v, table = _setup(B, L, Lq, Hq, Hkv, D, w_pre, w0, seed=123)
    kp, vp, bt = _paginate(k, v, L, ps, seed=124)
    good_o, good_l = _paged(w, qc, kp, vp, bt, table, Lq)
    bad_bt = bt.clone()
    slot = 5                                  # keys 640 .. 767
    bad_bt[1, slot] = kp.shape[0] + 3
    out, lse = _paged(w, qc, kp, vp, bad_bt, table, Lq)
    torch.cuda.synchronize()
    q_off = L - Lq
    pos = q_off + np.arange(Lq)
    BQ = 256 // (Hq // Hkv)                   # query positions per workgroup
    first_wg = q_off + ((slot * ps - q_off) // BQ) * BQ
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(o[0], good_o[0].cpu().numpy())          # the other sequence is untouched
    assert np.isnan(o[1][pos >= slot * ps]).all() and np.isnan(l[1][:, pos >= slot * ps]).all()
    keep = pos < first_wg                     # workgroups that never visit the page
    assert keep.any()
    assert np.array_equal(o[1][keep], good_o[1].cpu().numpy()[keep])


@pytest.mark.parametrize("Lq", [2, 16])
def test_out_of_range_page_on_the_decode_route(Lq):
    """Short chunks run on the decode kernels (2 tokens: the split kernel, 8
    columns; 16 tokens: the staged kernel, 4 column groups).  A block-table
    entry outside the pages poisons every row of its sequence (each row's keys
    include that page) and leaves the other sequence bit for bit as it was;
    the rows past L in the last page hold NaN and must not leak either."""
    require_gpu()
    B, L, Hq, Hkv, D, ps, w_pre, w0 = 2, 1000, 8, 2, 128, 128, 300, 64
    w, x, qc, k, v, table = _setup(B, L, Lq, Hq, Hkv, D, w_pre, w0, seed=321 + Lq)
    kp, vp, bt = _paginate(k, v, L, ps, seed=322 + Lq)
    good_o, good_l = _paged(w, qc, kp, vp, bt, table, Lq)
    ref_o, ref_l = _contig(w, qc, k, v, table, Lq)
    torch.cuda.synchronize()
    assert torch.isfinite(good_o).all()
    assert torch.equal(good_o, ref_o) and torch.equal(good_l, ref_l)
    bad_bt = bt.clone()
    bad_bt[1, 3] = kp.shape[0] + 7            # keys 384 .. 511, below every row of the chunk
    out, lse = _paged(w, qc, kp, vp, bad_bt, table, Lq)
    torch.cuda.synchronize()
    o, l = out.cpu().numpy(), lse.cpu().numpy()
    assert np.array_equal(o[0], good_o[0].cpu().numpy()) and np.array_equal(l[0], good_l[0].cpu().numpy())
    assert np.isnan(o[1]).all() and np.isnan(l[1]).all()
