"""Cache rows at positions >= L are not part of a call (Jet-Long §3.2: a step
at length L attends to keys 0..L-1 only), and a serving cache holds anything
there: rows not yet written, or a previous sequence's values.  With those
rows set to NaN, decode (contiguous and paged) and chunked prefill (on the
decode kernels and on the prefill kernels) give bit-identical results to the
same calls over a cache whose rows past L hold ordinary values."""
import numpy as np
import pytest
import torch

import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import require_gpu, to_dev
from test_gpu_paged import _paginate

pytestmark = pytest.mark.gpu

B, L, LMAX, HKV, D = 2, 517, 640, 2, 128   # 517 keys: ragged 32-key steps, odd step counts
HQ, W_PRE, W0, BASE = 4 * HKV, 256, 64, 1e4
SCALE = D ** -0.5


def _inputs(lq):
    rng = np.random.Generator(np.random.PCG64([L, 41]))
    bits = lambda shape: si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    kc, vc = to_dev(bits((B, LMAX, HKV, D)), "bf16"), to_dev(bits((B, LMAX, HKV, D)), "bf16")
    q = to_dev(bits((B, lq, HQ, D)), "bf16")
    kn, vn = kc.clone(), vc.clone()
    kn[:, L:] = float("nan")
    vn[:, L:] = float("nan")
    return q, kc, vc, kn, vn


def test_decode_ignores_rows_past_L():
    require_gpu()
    q, kc, vc, kn, vn = _inputs(1)
    table = jl.alloc_table(LMAX, D, BASE, w_pretrained=W_PRE)
    ws = jl.alloc_decode_workspace(B, HQ, D, LMAX)
    outs = []
    for k, v in ((kc, vc), (kn, vn)):
        out = torch.empty((B, 1, HQ, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, HQ), dtype=torch.float32, device="cuda")
        jl.jl_bifocal_decode(q, k, v, out, lse, L, W0, W_PRE, BASE, SCALE, table, ws)
        outs.append((out, lse))
    kp, vp, bt = _paginate(kn, vn, 64, seed=9)
    out = torch.empty((B, 1, HQ, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, HQ), dtype=torch.float32, device="cuda")
    jl.jl_bifocal_decode_paged(q, kp, vp, bt, out, lse, L, W0, W_PRE, BASE, SCALE, table, ws)
    outs.append((out, lse))
    torch.cuda.synchronize()
    assert torch.isfinite(outs[0][0]).all()
    for o, s in outs[1:]:
        assert torch.equal(o, outs[0][0]) and torch.equal(s, outs[0][1])


@pytest.mark.parametrize("lq", [4, 16, 100])   # decode split kernel, staged short-chunk kernel, prefill kernel
def test_chunk_ignores_rows_past_L(lq):
    require_gpu()
    q, kc, vc, kn, vn = _inputs(lq)
    table = jl.alloc_table(LMAX, D, BASE, w_pretrained=W_PRE)
    outs = []
    for k, v in ((kc, vc), (kn, vn)):
        out = torch.empty((B, lq, HQ, D), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((B, HQ, lq), dtype=torch.float32, device="cuda")
        jl.jl_bifocal_prefill_chunk(q, k, v, out, lse, L, W0, W_PRE, BASE, SCALE, table)
        outs.append((out, lse))
    torch.cuda.synchronize()
    print("lq", lq, "finite", bool(torch.isfinite(outs[0][0].float()).all()))
    assert torch.isfinite(outs[0][0].float()).all()
    assert torch.equal(outs[1][0], outs[0][0]) and torch.equal(outs[1][1], outs[0][1])
