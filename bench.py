"""Benchmark of the Jet-Long bifocal attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (seeded synthetic inputs, synth_inputs.py):
  * prefill: B=1, L=131072, 32 query / 8 KV heads, D=128, bf16, pretrained
    window 32768 (G=4), w0=4096, RoPE base 1e6 -- the 128K point;
  * decode: a bf16 cache of 131072 keys, then 256 steps of one new token
    each (L = 131073 .. 131328, G=5), same head shape.

A prefill step is one jl_bifocal_prefill call over the whole 128K sequence;
a decode step is one jl_bifocal_decode call (the new token's k/v rows are
written into the cache before timing, as the caller's projection would).  Inputs are resident in HBM before timing starts.  One
JSON line is printed: ``value`` is prefill TFLOP/s (algorithmic causal
FLOPs 4*B*Hq*D*L(L+1)/2 over the measured time); decode microseconds per
step and its HBM roofline ride in ``decode``; the CPU oracle is timed on a
bounded row sample in ``cpu_baseline``.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

METRIC = "bifocal prefill TFLOP/s @128K (% MFMA peak); decode µs/step @128K (% HBM BW)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, published (the device-derived peak rides beside it)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-passes", type=int, default=2, help="timed passes over the 256 decode steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=640, help="query rows in the CPU-oracle sample")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--chunk-steps", type=int, default=100,
                    help="timed calls per chunk length, after 3 untimed ones, in up to 5 batches whose "
                         "median mean is reported (0 skips the chunk leg)")
    ap.add_argument("--fi-steps", type=int, default=3,
                    help="timed calls of the prefill with the frequency-interpolation view (0: skip)")
    ap.add_argument("--unfused-steps", type=int, default=3,
                    help="calls of the unfused three-pass prefill timed (0 skips it)")
    ap.add_argument("--control-steps", type=int, default=5,
                    help="timed calls of the matched control (same inputs, every pair local); 0 skips it")
    ap.add_argument("--ref-secs", type=float, default=2.0,
                    help="seconds of each vendor reference (hipBLASLt bf16 GEMM, device copy) timed after the "
                         "library's legs; 0 skips them")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run one plain 512 MiB device-to-device copy (reference for HBM counters)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "traffic_prefill128k_decode128k.json")


def measured_traffic():
    """HBM bytes per dispatch from the committed PMC summary, keyed by kernel;
    empty if there is none or the library differs from the one it measured."""
    try:
        from zero_shot_rope_jl_amd.profiling import library_hash
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        if t.get("library_sha256") != library_hash():
            return {}
        return {k: (v["fetch_bytes"] or 0.0) + (v["write_bytes"] or 0.0) for k, v in t["kernels"].items()}
    except (OSError, ValueError, KeyError):
        return {}


# the kernels whose HBM traffic the roofline objects report (names as the
# profiler prints them)
PREFILL_KERNEL = "jl::prefill_bf16_kernel<128, true, 0, false>"
DECODE_KERNELS = ("jl::decode_split_kernel<128, true, false, false, false, false>", "jl::decode_combine_kernel<128, true>")


def pick(traffic, *prefixes):
    """Summed bytes per dispatch of the kernels whose names start with any of the prefixes."""
    hits = [v for k, v in traffic.items() if k.startswith(prefixes)]
    return sum(hits) if hits else None


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_dev(torch, arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def prefill_flops(w) -> float:
    return 4.0 * w.B * w.Hq * w.D * w.L * (w.L + 1) / 2.0


def bench_prefill(torch, jl, si, args, w, x):
    q, k, v = (to_dev(torch, x[n], w.dtype) for n in "qkv")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    ws = jl.alloc_prefill_workspace(k, w.w_pretrained)   # keys in their remote view (rewritten every step), tile counters
    torch.cuda.synchronize()

    def step():
        jl.jl_bifocal_prefill(q, k, v, out, lse, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] prefill warmup done, timing {args.steps} steps")
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    per_call = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    stats = {"mean": round(ms, 4), "median": round(float(np.median(per_call)), 4), "min": round(per_call[0], 4)}
    assert torch.isfinite(out[:, :: 4096].float()).all(), "non-finite prefill output"
    flops = prefill_flops(w)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] prefill {ms:.3f} ms/step (median {stats['median']:.3f}, min {stats['min']:.3f}), "
        f"{tflops:.1f} TFLOP/s (wall {wall:.2f}s)")
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    return ms, tflops, flops, stats


def bench_control(torch, jl, args, w, x):
    """The matched control: the same kernel on the same inputs with
    w_pretrained = L, so G = 1 and every pair is local (plain causal
    attention: no remote view, no rotation pre-pass, no window edge)."""
    q, k, v = (to_dev(torch, x[n], w.dtype) for n in "qkv")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    ws = jl.alloc_prefill_workspace(k, w.L)   # G = 1: the tile counters only

    def step():
        jl.jl_bifocal_prefill(q, k, v, out, lse, w.w0, w.L, w.rope_base, w.sm_scale, table, ws)

    step()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.control_steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.control_steps
    log(f"[bench] matched control (G=1) {ms:.3f} ms/call")
    del q, k, v, out, lse
    torch.cuda.empty_cache()
    return ms


def bench_unfused(torch, jl, args, w, x):
    """The same call computed unfused: three separate attention passes and
    their inclusion-exclusion merge (jl_bifocal_prefill_unfused)."""
    q, k, v = (to_dev(torch, x[n], w.dtype) for n in "qkv")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    table = jl.alloc_table(w.L, w.D, w.rope_base)
    ws = jl.alloc_prefill_unfused_workspace(q, k, w.w_pretrained)

    def step():
        jl.jl_bifocal_prefill_unfused(q, k, v, out, lse, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table,
                                      workspace=ws)

    step()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.unfused_steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.unfused_steps
    log(f"[bench] unfused (three passes + merge) {ms:.3f} ms/call")
    del q, k, v, out, lse, ws
    torch.cuda.empty_cache()
    return ms


FI_RAMP = (1.0, 32.0)   # YaRN's ramp bounds, in turns per pretrained window


def bench_fi(torch, jl, args, w, x):
    """The same call with the frequency-interpolation remote view
    (jl_bifocal_prefill_fi, YaRN's ramp bounds): its table build, then the
    prefill with the table in place."""
    q, k, v = (to_dev(torch, x[n], w.dtype) for n in "qkv")
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.L), dtype=torch.float32, device="cuda")
    ws = jl.alloc_prefill_workspace(k, w.w_pretrained)
    table = torch.empty(jl.jl_fi_table(w.L, w.w_pretrained, w.D, w.rope_base, *FI_RAMP), dtype=torch.uint8,
                        device="cuda")
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    jl.jl_fi_table(w.L, w.w_pretrained, w.D, w.rope_base, *FI_RAMP, table=table)
    torch.cuda.synchronize()
    ev0.record(stream)
    jl.jl_fi_table(w.L, w.w_pretrained, w.D, w.rope_base, *FI_RAMP, table=table)
    ev1.record(stream)
    torch.cuda.synchronize()
    table_ms = ev0.elapsed_time(ev1)

    def step():
        jl.jl_bifocal_prefill_fi(q, k, v, out, lse, w.w0, w.w_pretrained, w.rope_base, *FI_RAMP, w.sm_scale, table,
                                 workspace=ws)

    step()
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.fi_steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.fi_steps
    log(f"[bench] frequency-interpolation view: {ms:.3f} ms/call, table build {table_ms:.3f} ms")
    del q, k, v, out, lse, ws, table
    torch.cuda.empty_cache()
    return ms, table_ms


def bench_reorder(torch, jl, w, x):
    """jl_rope_interleaved_to_half over the workload's q and k (what a model
    with interleaved RoPE pairs adds per call), ms for both."""
    q, k = (to_dev(torch, x[n], w.dtype) for n in "qk")
    qo, ko = torch.empty_like(q), torch.empty_like(k)
    jl.jl_rope_interleaved_to_half(q, qo)
    jl.jl_rope_interleaved_to_half(k, ko)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(3):
        jl.jl_rope_interleaved_to_half(q, qo)
        jl.jl_rope_interleaved_to_half(k, ko)
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / 3
    gbs = 2.0 * (q.numel() + k.numel()) * q.element_size() / (ms * 1e-3) / 1e9
    log(f"[bench] interleaved-pair reorder of q and k: {ms:.3f} ms ({gbs:.0f} GB/s)")
    del q, k, qo, ko
    torch.cuda.empty_cache()
    return ms, gbs


CHUNK_LQ = (1, 16, 256, 4096)


def bench_chunk(torch, jl, args, w, x, page_size=256):
    """The last Lq tokens of the workload as one chunk over the cache of all L
    keys (jl_bifocal_prefill_chunk), for several chunk lengths.  Each length
    is timed as a chunk of a sequence prefilled chunk by chunk: the call's
    rotated-key state covers the rows before the chunk, so it rotates its own
    Lq new keys (the state is set back before every timed call).  The
    longest chunk is also timed without a state (every key rotated) and over
    the cache held in shuffled pages (jl_bifocal_prefill_chunk_paged)."""
    q, k, v = (to_dev(torch, x[n], w.dtype) for n in "qkv")
    table = jl.alloc_table(w.L, w.D, w.rope_base, w_pretrained=w.w_pretrained)
    G = (w.L + w.w_pretrained - 1) // w.w_pretrained
    max_pages = (w.L + page_size - 1) // page_size
    perm = np.random.Generator(np.random.PCG64([w.seed, 23])).permutation(w.B * max_pages)
    kp = torch.empty((w.B * max_pages, page_size, w.Hkv, w.D), dtype=k.dtype, device="cuda")
    vp = torch.empty_like(kp)
    for b in range(w.B):
        idx = torch.from_numpy(perm[b * max_pages:(b + 1) * max_pages].astype(np.int64)).cuda()
        kp[idx] = k[b].view(max_pages, page_size, w.Hkv, w.D)
        vp[idx] = v[b].view(max_pages, page_size, w.Hkv, w.D)
    bt = torch.from_numpy(perm.reshape(w.B, max_pages).astype(np.int32)).cuda()
    st = jl.alloc_chunk_state(q[:, :CHUNK_LQ[-1]], k, w.w_pretrained)
    # the state's rotated keys: every row, as the chunks before would have left them
    jl.jl_bifocal_prefill_chunk(q[:, -1:].contiguous(), k, v, torch.empty((w.B, 1, w.Hq, w.D), dtype=torch.bfloat16,
                                device="cuda"), None, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table,
                                workspace=st)
    assert (st.state.G, st.state.rows) == (G, w.L)
    stream = torch.cuda.current_stream()
    res = {}
    for Lq in CHUNK_LQ:
        qc = q[:, w.L - Lq:].contiguous()
        out = torch.empty((w.B, Lq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")

        def with_state():
            st.state.G, st.state.rows = G, w.L - Lq   # the earlier chunks rotated rows < L - Lq
            jl.jl_bifocal_prefill_chunk(qc, k, v, out, None, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale,
                                        table, workspace=st)
        calls = [(f"lq{Lq}_ms", with_state)]
        if Lq == CHUNK_LQ[-1]:
            calls.append((f"lq{Lq}_every_key_rotated_ms", lambda: jl.jl_bifocal_prefill_chunk(
                qc, k, v, out, None, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)))
            calls.append((f"lq{Lq}_paged_256_ms", lambda: jl.jl_bifocal_prefill_chunk_paged(
                qc, kp, vp, bt, out, None, w.L, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, table)))
        for name, call in calls:
            for _ in range(3):
                call()
            # the timed calls in batches back to back: a batch's mean per call can
            # swing by ~10% from one batch to the next, so the median batch is
            # reported
            batches = max(1, min(5, args.chunk_steps))
            per = max(1, args.chunk_steps // batches)
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 1)]
            torch.cuda.synchronize()
            evs[0].record(stream)
            for i in range(batches):
                for _ in range(per):
                    call()
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            means = [evs[i].elapsed_time(evs[i + 1]) / per for i in range(batches)]
            res[name] = round(float(np.median(means)), 4)
        del qc, out
    log("[bench] chunks over the 128K cache: " + ", ".join(f"{k} {v:.3f}" for k, v in res.items()))
    del q, k, v, kp, vp, st
    torch.cuda.empty_cache()
    return res


def bench_decode(torch, jl, si, args):
    dw = si.DECODE_WORKLOAD
    log(f"[bench] generating {dw.name} cache")
    kc_np, vc_np = si.make_decode_prompt(dw)
    kc, vc = to_dev(torch, kc_np, "bf16"), to_dev(torch, vc_np, "bf16")
    del kc_np, vc_np
    steps = [si.make_decode_step(dw, s) for s in range(1, dw.steps + 1)]
    qs = to_dev(torch, np.stack([s[0] for s in steps]), "bf16")     # [S, B, 1, Hq, D]
    ks = to_dev(torch, np.stack([s[1] for s in steps]), "bf16")
    vs = to_dev(torch, np.stack([s[2] for s in steps]), "bf16")
    table = jl.alloc_table(dw.Lmax, dw.D, dw.rope_base)
    ws = jl.alloc_decode_workspace(dw.B, dw.Hq, dw.D, dw.Lmax)
    out = torch.empty((dw.B, 1, dw.Hq, dw.D), dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()

    # Each step's new k/v row is written before timing: writing the row is the
    # caller's job (the projection that produces it), and step s reads only
    # rows < prompt_len + s, so rows of later steps do not change its result.
    kc[:, dw.prompt_len:dw.Lmax].copy_(ks[:, :, 0].transpose(0, 1))
    vc[:, dw.prompt_len:dw.Lmax].copy_(vs[:, :, 0].transpose(0, 1))

    def one_pass():
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode(qs[s], kc, vc, out, None, L, dw.w0, dw.w_pretrained, dw.rope_base,
                                 dw.sm_scale, table, ws)

    one_pass()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.decode_passes):
        one_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us = ev0.elapsed_time(ev1) * 1e3 / (args.decode_passes * dw.steps)
    # per-step median from one more pass with an event between steps (not part of the timed region)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(dw.steps + 1)]
    evs[0].record(stream)
    for s in range(dw.steps):
        L = dw.prompt_len + s + 1
        jl.jl_bifocal_decode(qs[s], kc, vc, out, None, L, dw.w0, dw.w_pretrained, dw.rope_base, dw.sm_scale, table, ws)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    us_median = float(np.median([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(dw.steps)]))

    # the matched control: the same kernel and steps with w_pretrained = Lmax,
    # so G = 1 and every key is read in its stored view
    def control_pass():
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode(qs[s], kc, vc, out, None, L, dw.w0, dw.Lmax, dw.rope_base, dw.sm_scale, table, ws)

    control_pass()
    ev0.record(stream)
    for _ in range(args.decode_passes):
        control_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_control = ev0.elapsed_time(ev1) * 1e3 / (args.decode_passes * dw.steps)

    # the unfused step: three decode passes (window in the stored view, every
    # key in the corrected view, window in the corrected view) and the §3.3
    # Eq. 6 merge
    uws = jl.alloc_decode_unfused_workspace(dw.B, dw.Hq, dw.D, dw.Lmax)
    uout = torch.empty_like(out)

    def unfused_pass():
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode_unfused(qs[s], kc, vc, uout, None, L, dw.w0, dw.w_pretrained, dw.rope_base,
                                         dw.sm_scale, table, uws)

    unfused_pass()
    ev0.record(stream)
    unfused_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_unfused = ev0.elapsed_time(ev1) * 1e3 / dw.steps
    one_pass()
    torch.cuda.synchronize()
    unfused_ok = bool((uout.float() - out.float()).abs().max().item() <= 2e-2)
    del uws, uout

    # the same steps over the cache held in shuffled 256-key pages
    ps = 256
    max_pages = (dw.Lmax + ps - 1) // ps
    perm = np.random.Generator(np.random.PCG64([dw.seed, 17])).permutation(dw.B * max_pages)
    kp = torch.zeros((dw.B * max_pages, ps, dw.Hkv, dw.D), dtype=kc.dtype, device="cuda")
    vp = torch.zeros_like(kp)
    for b in range(dw.B):
        for s in range(max_pages):
            rows = slice(s * ps, min((s + 1) * ps, dw.Lmax))
            kp[int(perm[b * max_pages + s]), : rows.stop - rows.start] = kc[b, rows]
            vp[int(perm[b * max_pages + s]), : rows.stop - rows.start] = vc[b, rows]
    bt = torch.from_numpy(perm.reshape(dw.B, max_pages).astype(np.int32)).cuda()

    def paged_pass():
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode_paged(qs[s], kp, vp, bt, out, None, L, dw.w0, dw.w_pretrained, dw.rope_base,
                                       dw.sm_scale, table, ws)

    paged_pass()
    ev0.record(stream)
    paged_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_paged = ev0.elapsed_time(ev1) * 1e3 / dw.steps
    del kp, vp

    # the 256 contiguous-cache steps captured once as a HIP graph and replayed;
    # the replay's last output must equal the eager pass's bit for bit
    one_pass()
    eager_out = out.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_pass()
    graph.replay()
    ev0.record(stream)
    graph.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_graph = ev0.elapsed_time(ev1) * 1e3 / dw.steps
    graph_ok = bool(torch.equal(out, eager_out))
    del graph

    # the same steps with the frequency-interpolation remote view (s from
    # each step's L, no table)
    def fi_pass():
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode_fi(qs[s], kc, vc, out, None, L, dw.w0, dw.w_pretrained, dw.rope_base, *FI_RAMP,
                                    dw.sm_scale, ws)

    fi_pass()
    ev0.record(stream)
    fi_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_fi = ev0.elapsed_time(ev1) * 1e3 / dw.steps

    # the same steps with a rotated-key cache: each timed pass starts from an
    # empty cache, so its first step rotates every remote key and the later
    # steps one new row each; that cost is inside the per-step figure
    rkc = jl.RotatedKeyCache(kc)

    def rkc_pass():
        rkc.reset()
        for s in range(dw.steps):
            L = dw.prompt_len + s + 1
            jl.jl_bifocal_decode_rkc(qs[s], kc, vc, rkc, out, None, L, dw.w0, dw.w_pretrained, dw.rope_base,
                                     dw.sm_scale, table, ws)

    rkc_pass()
    ev0.record(stream)
    for _ in range(args.decode_passes):
        rkc_pass()
    ev1.record(stream)
    torch.cuda.synchronize()
    us_rkc = ev0.elapsed_time(ev1) * 1e3 / (args.decode_passes * dw.steps)
    rkc_ok = bool((out.float() - eager_out.float()).abs().max().item() <= 2e-2)
    del rkc
    mean_L = dw.prompt_len + (dw.steps + 1) / 2.0
    bytes_step = 2.0 * dw.B * mean_L * dw.Hkv * dw.D * 2
    gbs = bytes_step / (us * 1e-6) / 1e9
    log(f"[bench] decode matched control (G=1) {us_control:.2f} us/step, unfused (three passes + merge) "
        f"{us_unfused:.2f} us/step{'' if unfused_ok else ' MISMATCH'}")
    log(f"[bench] decode {us:.2f} us/step (per-step median {us_median:.2f}, paged cache {us_paged:.2f}, "
        f"graph {us_graph:.2f}{'' if graph_ok else ' MISMATCH'}, rotated-key cache {us_rkc:.2f}, "
        f"frequency interpolation {us_fi:.2f}"
        f"{'' if rkc_ok else ' MISMATCH'}), {gbs:.0f} GB/s")
    del kc, vc
    torch.cuda.empty_cache()
    return dw, us, gbs, bytes_step, us_median, {"us_per_step_paged_256": round(us_paged, 3),
                                               "us_per_step_graph": round(us_graph, 3),
                                               "graph_matches_eager": graph_ok,
                                               "us_per_step_rotated_keys": round(us_rkc, 3),
                                               "us_per_step_frequency_interpolation": round(us_fi, 3),
                                               "rotated_keys_match": rkc_ok,
                                               "matched_control": {
                                                   "what": "same kernel and steps with w_pretrained = Lmax "
                                                           "(G = 1, every key in its stored view)",
                                                   "us_per_step": round(us_control, 3),
                                                   "bifocal_over_control": round(us_control / us, 4)},
                                               "unfused": {
                                                   "what": "three decode passes (stored view over the window, "
                                                           "corrected view over all keys and over the window) and "
                                                           "their inclusion-exclusion merge",
                                                   "us_per_step": round(us_unfused, 3),
                                                   "fused_speedup": round(us_unfused / us, 4),
                                                   "matches_fused": unfused_ok}}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads():
    """BLAS threads for the oracle: every core this process may run on."""
    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        return n, threadpool_limits(limits=n)
    except ImportError:  # pragma: no cover
        import contextlib
        return n, contextlib.nullcontext()


def cpu_baseline(si, w, x, n_rows):
    """The float64 oracle on a bounded sample of the same workload: all 32
    heads at n_rows seeded uniform query rows (all keys of each row), with
    the time for all L rows extrapolated by algorithmic FLOPs."""
    import oracle
    cores, limit = oracle_threads()
    f64 = (lambda a: si.f32_from_bf16_bits(a).astype(np.float64)) if w.dtype == "bf16" else \
        (lambda a: a.astype(np.float64))
    rng = np.random.Generator(np.random.PCG64([w.seed, 99]))
    rows = np.sort(rng.choice(w.L, size=n_rows, replace=False))
    q64 = np.zeros((w.B, w.L, w.Hq, w.D))
    q64[:, rows] = f64(x["q"][:, rows])
    k64, v64 = f64(x["k"]), f64(x["v"])
    with limit:
        t0 = time.perf_counter()
        oracle.bifocal_attention(q64, k64, v64, w.w0, w.w_pretrained, w.rope_base, w.sm_scale, rows=rows)
        sec = time.perf_counter() - t0
    flops = float(sum(4.0 * w.B * w.Hq * w.D * (r + 1) for r in rows))
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "rows_sampled": int(n_rows), "rows_total": int(w.L),
            "sample_s": round(sec, 2), "extrapolated_full_s": round(sec * prefill_flops(w) / flops, 1),
            "sample": f"{w.name}: {n_rows} seeded uniform query rows x all {w.Hq} heads over their causal keys "
                      f"(float64 NumPy oracle incl. the remote view of all {w.L} keys), {sec:.1f} s; the full "
                      f"{w.L}-row call extrapolated by algorithmic FLOPs"}


def cpu_baseline_decode(si, n_steps=2):
    """The float64 oracle on the first n_steps decode steps of the 128K-cache
    workload (one query token over every cached key per step)."""
    import oracle
    dw = si.DECODE_WORKLOAD
    cores, limit = oracle_threads()
    kc_np, vc_np = si.make_decode_prompt(dw)
    kc = si.f32_from_bf16_bits(kc_np).astype(np.float64)
    vc = si.f32_from_bf16_bits(vc_np).astype(np.float64)
    del kc_np, vc_np
    sec = 0.0
    with limit:
        for s in range(1, n_steps + 1):
            q, kn, vn = si.make_decode_step(dw, s)
            row = dw.prompt_len + s - 1
            kc[:, row] = si.f32_from_bf16_bits(kn[:, 0])
            vc[:, row] = si.f32_from_bf16_bits(vn[:, 0])
            q64 = si.f32_from_bf16_bits(q[:, 0]).astype(np.float64)
            t0 = time.perf_counter()
            oracle.decode_attention(q64, kc, vc, row + 1, dw.w0, dw.w_pretrained, dw.rope_base, dw.sm_scale)
            sec += time.perf_counter() - t0
    return {"value": sec / n_steps * 1e6, "unit": "µs/step", "cores": int(cores), "kind": "oracle",
            "cpu_model": cpu_model(), "steps_sampled": n_steps, "steps_total": dw.steps,
            "extrapolated_full_s": round(sec / n_steps * dw.steps, 1),
            "sample": f"{dw.name}: the first {n_steps} of its {dw.steps} steps (float64 NumPy oracle, every "
                      f"cached key incl. its remote view), {sec:.1f} s; all {dw.steps} steps extrapolated"}


def vendor_references(torch, secs: float) -> dict:
    """What the vendor's own code reaches on this GPU in the same run: a
    square bf16 GEMM (torch.matmul, i.e. hipBLASLt) on seeded N(0, 1) inputs
    like the workload's, and on zeros, each sustained for `secs` so the clock
    settles under load; and a 1 GiB device-to-device copy (read + write
    bytes per second).  They frame the published peaks: on random operands the
    shader clock is held down by power, on zeros it is not."""
    n = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    out = {}

    def sustained(fn, work):
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        reps = max(3, int(secs / max(time.perf_counter() - t, 1e-4)))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return work * reps / (e0.elapsed_time(e1) * 1e-3)

    for kind in ("random", "zeros"):
        if kind == "random":
            a = torch.randn(n, n, device="cuda", generator=g).bfloat16()
            b = torch.randn(n, n, device="cuda", generator=g).bfloat16()
        else:
            a = torch.zeros(n, n, device="cuda", dtype=torch.bfloat16)
            b = torch.zeros_like(a)
        c = torch.empty_like(a)
        out[f"gemm_bf16_{kind}_tflops"] = round(sustained(lambda: torch.matmul(a, b, out=c), 2.0 * n ** 3) / 1e12, 1)
        del a, b, c
    nb = 1 << 30
    src = torch.ones(nb, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    out["copy_gbs"] = round(sustained(lambda: dst.copy_(src), 2.0 * nb) / 1e9, 1)
    del src, dst
    out["what"] = (f"torch.matmul {n}x{n}x{n} bf16 (hipBLASLt) on seeded N(0,1) inputs and on zeros, and a "
                   f"{nb >> 30} GiB device copy (read + write bytes), each sustained ~{secs:g} s after the "
                   "library's legs")
    log(f"[bench] vendor references: {out}")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures a single GPU; --gpus {args.gpus} is not supported "
              "(every kernel here runs on one GPU's share of the work)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth_inputs as si
    import zero_shot_rope_jl_amd as jl
    assert torch.cuda.is_available(), "no GPU"
    log(f"[bench] library {jl.lib_path}")

    if args.copy_calibration:
        n = 512 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {n} bytes done")
        del src, dst
    n_cu, clk_khz = jl.jl_device_info(torch.cuda.current_device())
    peak_dev = n_cu * clk_khz * 1e3 * 4096 / 1e12
    log(f"[bench] device: {n_cu} CUs at {clk_khz / 1e6:.2f} GHz peak clock -> {peak_dev:.1f} TFLOP/s dense bf16")
    w = si.WORKLOADS["ext128k"]
    log(f"[bench] generating {w.name} inputs")
    x = si.make_prefill_inputs(w, want_f64=False)
    ms, tflops, flops, pstats = bench_prefill(torch, jl, si, args, w, x)
    traffic = measured_traffic()
    result = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "bifocal prefill, B1 L131072 Hq32 Hkv8 D128 bf16, w_pretrained 32768 (G=4), "
                               "w0 4096, RoPE base 1e6; decode: 131072-key cache + 256 steps (G=5)",
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": pick(traffic, PREFILL_KERNEL),
                     "flops_per_launch": flops,
                     "peak_device": round(peak_dev, 1), "frac_device": round(tflops / peak_dev, 4),
                     "peak_device_from": f"{n_cu} CUs x {clk_khz / 1e6:.2f} GHz x 4096 bf16 FLOP/clock/CU"},
        "prefill_ms_per_call": pstats,
    }
    if args.control_steps > 0:
        cms = bench_control(torch, jl, args, w, x)
        result["matched_control"] = {
            "what": "same kernel and inputs with w_pretrained = L (G = 1, every pair local)",
            "ms_per_call": round(cms, 4), "tflops": round(flops / (cms * 1e-3) / 1e12, 2),
            "bifocal_over_control": round(cms / ms, 4)}
    if args.unfused_steps > 0:
        ums = bench_unfused(torch, jl, args, w, x)
        result["unfused"] = {
            "what": "three separate passes (stored view over the window, corrected view over all keys and over "
                    "the window) and their inclusion-exclusion merge",
            "ms_per_call": round(ums, 4), "fused_speedup": round(ums / ms, 4)}
    if args.fi_steps > 0:
        fms, tms = bench_fi(torch, jl, args, w, x)
        result["frequency_interpolation"] = {
            "what": "same inputs, remote pairs in the YaRN-style frequency-interpolation view "
                    "(ramp bounds 1 and 32 turns per pretrained window)",
            "ms_per_call": round(fms, 4), "table_build_ms": round(tms, 4),
            "tflops": round(flops / (fms * 1e-3) / 1e12, 2)}
    if args.fi_steps > 0:
        rms, rgbs = bench_reorder(torch, jl, w, x)
        result["interleaved_reorder"] = {"what": "channel reorder of q and k for interleaved RoPE pairs",
                                         "ms_per_call": round(rms, 4), "gb_per_s": round(rgbs, 1)}
    if args.chunk_steps > 0:
        result["chunk"] = {"what": "the last Lq tokens of the workload as one chunk over all 131072 keys "
                                   f"(Lq = {', '.join(map(str, CHUNK_LQ))}), rotating its own Lq new keys (the "
                                   "rotated-key state covers the earlier rows); the longest also with every key "
                                   "rotated and over 256-key pages",
                           **bench_chunk(torch, jl, args, w, x)}
    if not args.skip_decode:
        dw, us, gbs, bytes_step, us_median, extra = bench_decode(torch, jl, si, args)
        result["decode"] = {
            "us_per_step": round(us, 3), "us_per_step_median": round(us_median, 3), **extra, "unit": "µs/step",
            "steps_timed": args.decode_passes * dw.steps,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": pick(traffic, *DECODE_KERNELS),
                         "bytes_per_step": bytes_step},
        }
    if "chunk" in result and "decode" in result and "lq16_ms" in result["chunk"]:
        # a 16-token chunk against one decode step over the same 128K cache
        result["chunk"]["lq16_over_decode_step"] = round(result["chunk"]["lq16_ms"] * 1e3 /
                                                         result["decode"]["us_per_step"], 3)
    if args.ref_secs > 0:
        ref = vendor_references(torch, args.ref_secs)
        result["vendor_reference"] = ref
        result["roofline"]["frac_of_vendor_gemm_random"] = round(tflops / ref["gemm_bf16_random_tflops"], 4)
        if "decode" in result:
            result["decode"]["roofline"]["frac_of_vendor_copy"] = round(
                result["decode"]["roofline"]["achieved"] / ref["copy_gbs"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(si, w, x, args.cpu_rows)
        if not args.skip_decode:
            result["cpu_baseline_decode"] = cpu_baseline_decode(si)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
