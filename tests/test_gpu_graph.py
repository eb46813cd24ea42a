"""HIP-graph capture of the library's calls: a graph holding a prefill and
several decode steps (contiguous and paged caches) replays to the same bits
as the eager calls, replay after replay, with other eager work on the same
workspace and outputs in between.  The calls launch kernels only (no
memsets, no synchronisation), so they can be captured."""
import numpy as np
import pytest
import torch

import synth_inputs as si
import zero_shot_rope_jl_amd as jl
from gpu_common import require_gpu, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    require_gpu()
    B, Lp, Hq, Hkv, D, w_pre, w0, base = 1, 1500, 8, 2, 128, 512, 100, 1e4
    scale, steps, ps = D ** -0.5, 4, 64
    Lmax = Lp + steps
    rng = np.random.Generator(np.random.PCG64([2024, 1]))
    bf = lambda *shape: to_dev(si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32)), "bf16")
    q, k, v = bf(B, Lp, Hq, D), bf(B, Lp, Hkv, D), bf(B, Lp, Hkv, D)
    kc, vc = bf(B, Lmax, Hkv, D), bf(B, Lmax, Hkv, D)
    qs = [bf(B, 1, Hq, D) for _ in range(steps + 1)]
    table = jl.alloc_table(Lmax, D, base)
    pws = jl.alloc_prefill_workspace(k, w_pre)
    dws = jl.alloc_decode_workspace(B, Hq, D, Lmax)
    # the same cache in shuffled pages
    mp = (Lmax + ps - 1) // ps
    perm = rng.permutation(B * mp)
    kp = torch.zeros((B * mp, ps, Hkv, D), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    for s in range(mp):
        n = min(ps, Lmax - s * ps)
        kp[int(perm[s]), :n] = kc[0, s * ps:s * ps + n]
        vp[int(perm[s]), :n] = vc[0, s * ps:s * ps + n]
    bt = torch.from_numpy(perm.reshape(B, mp).astype(np.int32)).cuda()

    pout = torch.empty((B, Lp, Hq, D), dtype=torch.bfloat16, device="cuda")
    plse = torch.empty((B, Hq, Lp), dtype=torch.float32, device="cuda")
    douts = [torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda") for _ in range(2 * steps)]
    dlses = [torch.empty((B, Hq), dtype=torch.float32, device="cuda") for _ in range(2 * steps)]

    def calls():
        jl.jl_bifocal_prefill(q, k, v, pout, plse, w0, w_pre, base, scale, table, workspace=pws)
        for s in range(steps):
            L = Lp + s + 1
            jl.jl_bifocal_decode(qs[s], kc, vc, douts[s], dlses[s], L, w0, w_pre, base, scale, table, dws)
            jl.jl_bifocal_decode_paged(qs[s], kp, vp, bt, douts[steps + s], dlses[steps + s], L, w0, w_pre,
                                       base, scale, table, dws)

    calls()
    torch.cuda.synchronize()
    want = [t.clone() for t in [pout, plse, *douts, *dlses]]
    assert all(torch.isfinite(t.float()).all() for t in want)
    for s in range(steps):   # paged and contiguous agree bit for bit
        assert torch.equal(want[2 + s], want[2 + steps + s])

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    other = torch.empty((B, 1, Hq, D), dtype=torch.float32, device="cuda")
    for r in range(3):
        for t in [pout, plse, *douts, *dlses]:
            t.zero_()
        # unrelated eager work on the same workspaces between replays
        jl.jl_bifocal_decode(qs[steps], kc, vc, other, None, Lmax, w0, w_pre, base, scale, table, dws)
        jl.jl_bifocal_prefill(q[:, :700].contiguous(), k[:, :700].contiguous(), v[:, :700].contiguous(),
                              torch.empty((B, 700, Hq, D), dtype=torch.bfloat16, device="cuda"), None,
                              w0, w_pre, base, scale, table, workspace=pws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [pout, plse, *douts, *dlses]
        bad = [i for i, (g, w) in enumerate(zip(got, want)) if not torch.equal(g, w)]
        print("replay", r, "mismatched tensors", bad)
        assert not bad


def test_graph_replays_of_a_prefill_on_the_dynamic_grid():
    """A prefill large enough for the dynamic grid (its static grid would take
    more than two rounds of workgroups: 1024 query tiles here) holds a launch
    that clears its tile counters before the attention kernel; captured in a
    graph, every replay must clear them again and compute every tile.  The
    outputs are filled with NaN before each replay, so a replay that skipped
    tiles would leave NaN behind; every replay must equal the eager call bit
    for bit, with an eager call on the same workspace in between."""
    require_gpu()
    B, L, Hq, Hkv, D, w_pre, w0, base = 1, 8192, 32, 8, 128, 2048, 512, 1e6
    scale = D ** -0.5
    n_tiles = (L // (256 // (Hq // Hkv))) * Hkv * B
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    print(f"[graph] {n_tiles} query tiles over {n_cu} compute units", flush=True)
    assert n_tiles > 2 * n_cu
    rng = np.random.Generator(np.random.PCG64([2024, 2]))
    bf = lambda *shape: to_dev(si.bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32)), "bf16")
    q, k, v = bf(B, L, Hq, D), bf(B, L, Hkv, D), bf(B, L, Hkv, D)
    table = jl.alloc_table(L, D, base)
    ws = jl.alloc_prefill_workspace(k, w_pre)
    out = torch.empty((B, L, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq, L), dtype=torch.float32, device="cuda")

    def call():
        jl.jl_bifocal_prefill(q, k, v, out, lse, w0, w_pre, base, scale, table, workspace=ws)

    call()
    torch.cuda.synchronize()
    want_out, want_lse = out.clone(), lse.clone()
    assert torch.isfinite(want_out.float()).all() and torch.isfinite(want_lse).all()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for r in range(3):
        call()   # eager work on the same workspace (its counters end exhausted)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, want_out) and torch.equal(lse, want_lse)
        print(f"[graph] dynamic-grid prefill replay {r}: equal to the eager call: {same}", flush=True)
        assert same
