"""GPU check of jl_rope_interleaved_to_half: the reorder is bit-exact, and a
prefill over q and k reordered from interleaved RoPE pairs matches the
oracle on the same reordered vectors, which the CPU pins tie to scalar loops
written for interleaved pairs."""
import numpy as np
import pytest
import torch

import oracle
import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import TOL_BF16, max_err, prefill, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype,D,rows", [(torch.bfloat16, 128, 1000), (torch.float32, 64, 777),
                                          (torch.bfloat16, 64, 1)])
def test_reorder_is_bit_exact(dtype, D, rows):
    require_gpu()
    g = torch.Generator(device="cuda").manual_seed(rows)
    x = torch.randn(rows, D, device="cuda", generator=g).to(dtype)
    out = jl.jl_rope_interleaved_to_half(x)
    torch.cuda.synchronize()
    want = torch.cat([x[:, 0::2], x[:, 1::2]], dim=1)
    assert torch.equal(out, want)


def test_prefill_over_reordered_inputs_matches_oracle():
    require_gpu()
    w = si.Workload("ilv", "bf16", 1, 1000, 8, 2, 128, 64, 300, 1e4, 41)
    x = si.make_prefill_inputs(w)
    q, k, v = (to_dev(x[n], "bf16") for n in "qkv")           # read as interleaved-RoPE vectors
    qh, kh = jl.jl_rope_interleaved_to_half(q), jl.jl_rope_interleaved_to_half(k)
    out, lse = prefill(qh, kh, v, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, torch.float32)
    torch.cuda.synchronize()
    perm = [2 * j for j in range(w.D // 2)] + [2 * j + 1 for j in range(w.D // 2)]
    ref, ref_lse = oracle.bifocal_attention(x["q64"][..., perm], x["k64"][..., perm], x["v64"], w.w0,
                                            w.w_pretrained, w.rope_base, w.sm_scale)
    e, el = max_err(out.cpu().numpy(), ref), max_err(lse.cpu().numpy(), ref_lse)
    print("interleaved model err", e, "lse", el)
    assert e <= TOL_BF16 and el <= TOL_BF16
