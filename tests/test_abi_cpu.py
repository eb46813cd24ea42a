"""CPU checks of libjetlong.so: it loads, exports every symbol the header
declares, rejects bad arguments before touching HIP, computes G, and builds
the correction table exactly as an independent NumPy float64 computation."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import zero_shot_rope_jl_amd as jl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000   # aligned, never dereferenced: every call below fails validation


def header_symbols():
    with open(os.path.join(ROOT, "include", "jetlong.h")) as fh:
        txt = fh.read()
    return sorted(set(re.findall(r"JL_API\s+[\w\s\*]+?\b(jl_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol():
    syms = header_symbols()
    assert syms == sorted(["jl_last_error", "jl_version", "jl_schedule", "jl_bifocal_prefill_workspace",
                           "jl_bifocal_prefill", "jl_bifocal_prefill_chunk", "jl_bifocal_decode_workspace",
                           "jl_bifocal_decode", "jl_bifocal_decode_paged", "jl_table_fill_host",
                           "jl_bifocal_prefill_unfused_workspace", "jl_bifocal_prefill_unfused",
                           "jl_bifocal_prefill_chunk_paged", "jl_bifocal_decode_rkc", "jl_fi_table",
                           "jl_fi_table_fill_host", "jl_bifocal_prefill_fi", "jl_bifocal_decode_fi",
                           "jl_rope_interleaved_to_half", "jl_bifocal_decode_unfused_workspace",
                           "jl_bifocal_decode_unfused", "jl_device_info", "jl_bifocal_decode_noalloc",
                           "jl_bifocal_prefill_chunk_workspace"])
    for s in syms:
        assert hasattr(jl.lib, s), s
    assert jl.jl_version() == 13


def test_schedule_golden_and_table_size():
    with open(os.path.join(ROOT, "tests", "golden", "schedule_examples.json")) as fh:
        for e in json.load(fh)["examples"]:
            G, need = jl.jl_schedule(e["L"], e["w_pretrained"], 128, 1e6)
            assert G == e["G"], e["cite"]
            # two levels: 1024 low rows, then one high row per 1024 offsets below
            # n(L-1) + 1, where n(p) = p - floor(p/G) (the largest offset a call reads)
            n_cover = (e["L"] - 1) - (e["L"] - 1) // G + 1
            assert need == 64 + (1024 + -(-n_cover // 1024)) * 64 * 8


def test_table_is_small_at_one_million_tokens():
    """A 1M-token call extended 4x (w_pretrained 256K, G = 4) reads offsets below
    786433: the table is under 1 MB at D = 128."""
    G, need = jl.jl_schedule(1 << 20, 1 << 18, 128, 1e6)
    assert G == 4 and need == 64 + (1024 + 769) * 512 and need < 1_000_000
    # without the pretrained window (w_pretrained = 1: G = L, offsets up to L - 1)
    _, worst = jl.jl_schedule(1 << 20, 1, 128, 1e6)
    assert worst == 64 + 2048 * 512


def _sched(L=100, w=10, D=128, base=1e4, G=True, table=None, tbytes=0):
    g = ctypes.c_int64(-7)
    need = ctypes.c_size_t(0)
    rc = jl.lib.jl_schedule(L, w, D, base, ctypes.byref(g) if G else None, table, tbytes,
                            ctypes.byref(need), None)
    return rc, g.value


@pytest.mark.parametrize("kw,code", [
    (dict(L=0), jl.JL_EINVAL), (dict(w=0), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
    (dict(base=1.0), jl.JL_EINVAL), (dict(base=float("nan")), jl.JL_EINVAL), (dict(G=False), jl.JL_EINVAL),
    (dict(table=FAKE, tbytes=10), jl.JL_ESPACE), (dict(table=FAKE + 4, tbytes=1 << 30), jl.JL_EINVAL),
])
def test_schedule_validation(kw, code):
    rc, g = _sched(**kw)
    assert rc == code
    assert jl.jl_last_error()
    assert g == -7            # output untouched


def _prefill(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=256, Hq=4,
             Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_prefill(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                     a["L"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"], a["base"],
                                     a["sc"], a["table"], a["tb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q=None), jl.JL_EINVAL), (dict(table=None), jl.JL_EINVAL), (dict(out=FAKE + 2), jl.JL_EINVAL),
    (dict(lse=FAKE + 4), jl.JL_EINVAL), (dict(B=0), jl.JL_EINVAL), (dict(L=0), jl.JL_EINVAL),
    (dict(Hq=3), jl.JL_EINVAL), (dict(w0=-1), jl.JL_EINVAL), (dict(wp=0), jl.JL_EINVAL),
    (dict(sc=0.0), jl.JL_EINVAL), (dict(sc=float("inf")), jl.JL_EINVAL), (dict(i=5), jl.JL_EINVAL),
    (dict(L=(1 << 30) + 1), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
    (dict(i=jl.JL_F32, o=jl.JL_BF16), jl.JL_EUNSUPPORTED), (dict(Hq=32, Hkv=2), jl.JL_EUNSUPPORTED),
    (dict(Hq=6, Hkv=2), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE), (dict(base=0.5), jl.JL_EINVAL),
    (dict(ws=None), jl.JL_ESPACE), (dict(wsb=256 * 2 * 128 * 2 - 1), jl.JL_ESPACE), (dict(ws=FAKE + 8), jl.JL_EINVAL),
])
def test_prefill_validation(over, code):
    assert _prefill(**over) == code
    assert jl.jl_last_error()


def test_prefill_workspace_size():
    up = lambda x: (x + 255) // 256 * 256
    sched = 8 * 128   # eight tile counters of the bf16 kernel's dynamic grid, one 128-byte line each
    # bf16 with G = ceil(L / w_pretrained) > 1: the keys in their remote view, B*L*Hkv*D bf16, then the counters
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 1, 131072, 8, 128, 32768) == 131072 * 8 * 128 * 2 + sched
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 2, 300, 2, 64, 256) == up(2 * 300 * 2 * 64 * 2) + sched
    # bf16 with G == 1 (every pair local): the counters only; fp32 inputs: none
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 1, 4096, 8, 128, 4096) == sched
    assert jl.jl_bifocal_prefill_workspace(jl.JL_F32, 1, 131072, 8, 128, 32768) == 0
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 1, 10, 1, 96, 4)
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 0, 10, 1, 64, 4)


def test_prefill_without_workspace_when_none_is_needed_passes_validation_order():
    # G == 1: a NULL workspace is accepted; the call still fails later, on the
    # unsupported head_dim, before any HIP call
    assert _prefill(L=64, wp=64, ws=None, wsb=0, D=96) == jl.JL_EUNSUPPORTED


def _unfused(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=256, Hq=4,
             Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_prefill_unfused(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                             a["L"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"], a["base"],
                                             a["sc"], a["table"], a["tb"], a["ws"], a["wsb"], None)


# bf16, B 1, L 256, Hq 4, Hkv 2, D 128, w_pretrained 64 (G = 4): rotated keys
# 256*2*128*2 B, then three fp32 outputs of 256*4*128*4 B, three fp32
# log-sum-exps of 4*256*4 B (every part a multiple of 256 B already) and the
# eight 128-byte tile counters of the bf16 kernel's dynamic grid
UNFUSED_WS = 256 * 2 * 128 * 2 + 3 * 256 * 4 * 128 * 4 + 3 * 4 * 256 * 4 + 8 * 128


@pytest.mark.parametrize("over,code", [
    (dict(q=None), jl.JL_EINVAL), (dict(table=None), jl.JL_EINVAL), (dict(out=FAKE + 2), jl.JL_EINVAL),
    (dict(lse=FAKE + 4), jl.JL_EINVAL), (dict(B=0), jl.JL_EINVAL), (dict(L=0), jl.JL_EINVAL),
    (dict(Hq=3), jl.JL_EINVAL), (dict(w0=-1), jl.JL_EINVAL), (dict(wp=0), jl.JL_EINVAL),
    (dict(sc=0.0), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED), (dict(i=jl.JL_F32, o=jl.JL_BF16),
                                                                     jl.JL_EUNSUPPORTED),
    (dict(Hq=32, Hkv=2), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE), (dict(ws=None), jl.JL_EINVAL),
    (dict(wsb=UNFUSED_WS - 1), jl.JL_ESPACE), (dict(ws=FAKE + 8), jl.JL_EINVAL),
])
def test_prefill_unfused_validation(over, code):
    assert _unfused(**over) == code
    assert jl.jl_last_error()


def test_prefill_unfused_workspace_size():
    assert jl.jl_bifocal_prefill_unfused_workspace(jl.JL_BF16, 1, 256, 4, 2, 128, 64) == UNFUSED_WS
    # fp32 inputs: no rotated keys; 100 rows: 3 * 100*8*64*4 B outputs and
    # 3 * 8*100*4 B = 3200 B log-sum-exps, each rounded up to 256 B (3328)
    assert jl.jl_bifocal_prefill_unfused_workspace(jl.JL_F32, 1, 100, 8, 2, 64, 64) == 3 * 204800 + 3 * 3328
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_prefill_unfused_workspace(jl.JL_BF16, 1, 10, 0, 1, 64, 4)


def _chunk(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, Lq=64, L=600,
             Lmax=700, Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE,
             wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_prefill_chunk(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                           a["Lq"], a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["w0"],
                                           a["wp"], a["base"], a["sc"], a["table"], a["tb"], a["ws"], a["wsb"],
                                           a.get("state"), None)


@pytest.mark.parametrize("over,code", [
    (dict(Lq=0), jl.JL_EINVAL), (dict(Lq=601), jl.JL_EINVAL), (dict(Lmax=599), jl.JL_EINVAL),
    (dict(L=0), jl.JL_EINVAL), (dict(q=None), jl.JL_EINVAL), (dict(out=FAKE + 2), jl.JL_EINVAL),
    (dict(D=96), jl.JL_EUNSUPPORTED), (dict(Hq=32, Hkv=2), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE),
    (dict(ws=None), jl.JL_ESPACE), (dict(wsb=700 * 2 * 128 * 2 - 1), jl.JL_ESPACE),
    (dict(i=jl.JL_F32, o=jl.JL_BF16), jl.JL_EUNSUPPORTED), (dict(Lmax=(1 << 30) + 1), jl.JL_EINVAL),
    (dict(state=ctypes.pointer(jl.JLRotatedKeys(4, 701))), jl.JL_EINVAL),
    (dict(state=ctypes.pointer(jl.JLRotatedKeys(4, -1))), jl.JL_EINVAL),
])
def test_prefill_chunk_validation(over, code):
    assert _chunk(**over) == code
    assert jl.jl_last_error()


def _chunk_paged(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, Lq=64, L=600,
             npg=10, ps=128, mp=5, Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30,
             ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_prefill_chunk_paged(a["q"], a["k"], a["v"], a["bt"], a["out"], a["lse"], a["i"],
                                                 a["o"], a["B"], a["Lq"], a["L"], a["npg"], a["ps"], a["mp"],
                                                 a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"], a["base"], a["sc"],
                                                 a["table"], a["tb"], a["ws"], a["wsb"], a.get("state"), None)


@pytest.mark.parametrize("over,code", [
    (dict(bt=None), jl.JL_EINVAL), (dict(bt=FAKE + 2), jl.JL_EINVAL), (dict(ps=64), jl.JL_EINVAL),
    (dict(ps=192), jl.JL_EINVAL), (dict(ps=0), jl.JL_EINVAL), (dict(npg=0), jl.JL_EINVAL),
    (dict(mp=4), jl.JL_EINVAL), (dict(mp=0), jl.JL_EINVAL), (dict(Lq=0), jl.JL_EINVAL),
    (dict(Lq=601), jl.JL_EINVAL), (dict(q=None), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
    (dict(i=jl.JL_F32, o=jl.JL_F32), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE),
    (dict(ws=None), jl.JL_ESPACE), (dict(wsb=640 * 2 * 128 * 2 - 1), jl.JL_ESPACE),
    (dict(mp=(1 << 23) + 1), jl.JL_EINVAL),
])
def test_prefill_chunk_paged_validation(over, code):
    assert _chunk_paged(**over) == code
    assert jl.jl_last_error()


def _decode_rkc(state, **over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, kr=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=600, Lmax=700,
             Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_decode_rkc(a["q"], a["k"], a["v"], a["kr"], state, a["out"], a["lse"], a["i"], a["o"],
                                        a["B"], a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"],
                                        a["base"], a["sc"], a["table"], a["tb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,rows,code", [
    (dict(kr=None), 0, jl.JL_EINVAL), (dict(kr=FAKE + 8), 0, jl.JL_EINVAL), (dict(), -1, jl.JL_EINVAL),
    (dict(), 701, jl.JL_EINVAL), (dict(Lmax=599), 0, jl.JL_EINVAL), (dict(ws=None), 0, jl.JL_EINVAL),
    (dict(i=jl.JL_F32, o=jl.JL_F32), 0, jl.JL_EUNSUPPORTED), (dict(tb=100), 0, jl.JL_ESPACE),
])
def test_decode_rkc_validation_leaves_state_alone(over, rows, code):
    st = jl.JLRotatedKeys(3, rows)
    assert _decode_rkc(ctypes.byref(st), **over) == code
    assert jl.jl_last_error()
    assert (st.G, st.rows) == (3, rows)


def test_decode_rkc_null_state():
    assert _decode_rkc(None) == jl.JL_EINVAL


def _decode(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=600, Lmax=700,
             Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE,
             wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_decode(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                    a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"],
                                    a["base"], a["sc"], a["table"], a["tb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(ws=None), jl.JL_EINVAL), (dict(Lmax=599), jl.JL_EINVAL), (dict(i=jl.JL_F32, o=jl.JL_F32),
                                                                    jl.JL_EUNSUPPORTED),
    (dict(Hq=64, Hkv=2), jl.JL_EUNSUPPORTED), (dict(wsb=16), jl.JL_ESPACE), (dict(tb=64), jl.JL_ESPACE),
    (dict(w0=-3), jl.JL_EINVAL), (dict(D=32), jl.JL_EUNSUPPORTED), (dict(k=FAKE + 8), jl.JL_EINVAL),
    (dict(Hq=6, Hkv=3), jl.JL_EUNSUPPORTED),
])
def test_decode_validation(over, code):
    assert _decode(**over) == code
    assert jl.jl_last_error()


def _paged(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=2, L=600,
             n_pages=40, ps=64, mp=10, Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE,
             tb=1 << 30, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_decode_paged(a["q"], a["k"], a["v"], a["bt"], a["out"], a["lse"], a["i"], a["o"],
                                          a["B"], a["L"], a["n_pages"], a["ps"], a["mp"], a["Hq"], a["Hkv"],
                                          a["D"], a["w0"], a["wp"], a["base"], a["sc"], a["table"], a["tb"],
                                          a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(bt=None), jl.JL_EINVAL), (dict(bt=FAKE + 2), jl.JL_EINVAL), (dict(ps=48), jl.JL_EINVAL),
    (dict(ps=0), jl.JL_EINVAL), (dict(mp=9), jl.JL_EINVAL), (dict(n_pages=0), jl.JL_EINVAL),
    (dict(i=jl.JL_F32, o=jl.JL_F32), jl.JL_EUNSUPPORTED), (dict(wsb=16), jl.JL_ESPACE),
    (dict(k=None), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
])
def test_decode_paged_validation(over, code):
    assert _paged(**over) == code
    assert jl.jl_last_error()


def _up(x):
    return (x + 255) // 256 * 256


def _dec_ws(B, Hq, D, splits):
    """Split partials [B, Hq, splits, D + 2] fp32."""
    return B * Hq * splits * (D + 2) * 4


def test_decode_workspace_size():
    assert jl.jl_bifocal_decode_workspace(1, 32, 128, 131328) == _dec_ws(1, 32, 128, 256)
    assert jl.jl_bifocal_decode_workspace(1, 32, 128, 1000) == _dec_ws(1, 32, 128, 32)
    assert jl.jl_bifocal_decode_workspace(2, 4, 64, 1) == _dec_ws(2, 4, 64, 1)
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_decode_workspace(1, 4, 96, 10)


def test_decode_unfused_workspace_size():
    base = _up(_dec_ws(1, 32, 128, 256))
    assert jl.jl_bifocal_decode_unfused_workspace(1, 32, 128, 131328) == \
        base + 3 * _up(32 * 128 * 4) + 3 * _up(32 * 4)
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_decode_unfused_workspace(0, 4, 128, 10)


def _unfused_dec(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=600, Lmax=700,
             Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE,
             wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_decode_unfused(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                            a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"],
                                            a["base"], a["sc"], a["table"], a["tb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(ws=None), jl.JL_EINVAL), (dict(Lmax=599), jl.JL_EINVAL), (dict(i=jl.JL_F32, o=jl.JL_F32),
                                                                    jl.JL_EUNSUPPORTED),
    (dict(wsb=jl.jl_bifocal_decode_workspace(1, 8, 128, 600)), jl.JL_ESPACE), (dict(tb=64), jl.JL_ESPACE),
    (dict(w0=-1), jl.JL_EINVAL), (dict(table=None), jl.JL_EINVAL),
])
def test_decode_unfused_validation(over, code):
    """The unfused step needs room for the fused step's workspace and its
    three pass results; anything less is refused before any HIP call."""
    assert _unfused_dec(**over) == code
    assert jl.jl_last_error()


@pytest.mark.parametrize("D,base,L", [(64, 1e4, 512), (128, 1e6, 131328), (128, 5e5, 1)])
def test_host_table_matches_numpy_float64(D, base, L):
    buf = jl.jl_table_fill_host(L, D, base)
    hdr = buf[:64]
    assert hdr[:4].view(np.uint32)[0] == 0x324C544A
    assert hdr[4:8].view(np.int32)[0] == D
    assert hdr[8:16].view(np.int64)[0] == L
    assert hdr[16:24].view(np.float64)[0] == base
    n_hi = -(-L // 1024)
    ent = buf[64:].view(np.float32).reshape(1024 + n_hi, D // 2, 2)
    theta = base ** (-(2.0 * np.arange(D // 2)) / D)          # independent float64 definition
    # the rows: angles l * theta (l < 1024), then 1024 h * theta (h < ceil(L / 1024))
    mult = np.concatenate([np.arange(1024), 1024 * np.arange(n_hi)]).astype(np.float64)
    ang = mult[:, None] * theta[None, :]
    want = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    # one fp32 ulp of rounding plus the float64 angle error (|n * d(theta)| < 1e-10)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ent.astype(np.float64) - want) <= ulp + 1e-10)
    # the entry of offset n is TL[n mod 1024] * TH[n / 1024]: within a few fp32
    # ulp of (cos, sin)(n theta) for every n the table covers
    n = np.unique(np.concatenate([np.arange(min(L, 2100)), np.random.default_rng(L).integers(0, L, 2000)]))
    n = n[n < L]
    lo, hi = ent[n % 1024].astype(np.float64), ent[1024 + n // 1024].astype(np.float64)
    c = lo[..., 0] * hi[..., 0] - lo[..., 1] * hi[..., 1]
    s_ = lo[..., 0] * hi[..., 1] + lo[..., 1] * hi[..., 0]
    a = n[:, None].astype(np.float64) * theta[None, :]
    assert np.max(np.abs(c - np.cos(a))) <= 4e-7 and np.max(np.abs(s_ - np.sin(a))) <= 4e-7


def test_binding_has_no_cpu_fallback():
    import zero_shot_rope_jl_amd.binding as b
    src = open(b.__file__).read()
    assert "oracle" not in src and "numpy.einsum" not in src and "softmax" not in src


def test_single_hip_runtime_in_process():
    # the library must bind to the HIP runtime torch already loaded: two
    # runtimes in one process leave the second without a device
    with open("/proc/self/maps") as fh:
        libs = {l.split()[-1] for l in fh if "libamdhip64" in l}
    assert len(libs) == 1, libs


# ---- frequency-interpolation view ------------------------------------------
@pytest.mark.parametrize("D,base,L,w_pre,alpha,beta", [
    (64, 1e4, 512, 256, 1.0, 32.0), (128, 1e6, 131328, 32768, 1.0, 32.0), (128, 5e5, 300, 1000, 1.0, 32.0),
    (128, 1e4, 1000, 100, -2.0, -1.0), (64, 1e4, 777, 64, 50.0, 100.0)])
def test_host_fi_table_matches_oracle(D, base, L, w_pre, alpha, beta):
    """Rows p of (cos, sin)(p (theta_i - theta'_i)), theta' from the oracle."""
    import oracle
    buf = jl.jl_fi_table_fill_host(L, w_pre, D, base, alpha, beta)
    hdr = buf[:64]
    assert hdr[:4].view(np.uint32)[0] == 0x3146544A
    assert hdr[4:8].view(np.int32)[0] == D and hdr[8:16].view(np.int64)[0] == L
    assert hdr[16:24].view(np.float64)[0] == base
    assert hdr[24:32].view(np.int64)[0] == L and hdr[32:40].view(np.int64)[0] == w_pre
    assert hdr[40:48].view(np.float64)[0] == alpha and hdr[48:56].view(np.float64)[0] == beta
    n_hi = -(-L // 1024)
    ent = buf[64:].view(np.float32).reshape(1024 + n_hi, D // 2, 2)
    phi = oracle.inv_freq(D, base) - oracle.fi_inv_freq(D, base, L, w_pre, alpha, beta)
    mult = np.concatenate([np.arange(1024), 1024 * np.arange(n_hi)]).astype(np.float64)
    ang = mult[:, None] * phi[None, :]
    want = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ent.astype(np.float64) - want) <= ulp + 1e-10)
    # position p: TL[p mod 1024] * TH[p / 1024] within a few fp32 ulp of (cos, sin)(p phi)
    p = np.arange(L)
    lo, hi = ent[p % 1024].astype(np.float64), ent[1024 + p // 1024].astype(np.float64)
    a = p[:, None].astype(np.float64) * phi[None, :]
    assert np.max(np.abs(lo[..., 0] * hi[..., 0] - lo[..., 1] * hi[..., 1] - np.cos(a))) <= 4e-7
    assert np.max(np.abs(lo[..., 0] * hi[..., 1] + lo[..., 1] * hi[..., 0] - np.sin(a))) <= 4e-7
    if L <= w_pre or alpha < 0:   # s = 1, or every pair kept: the identity
        assert np.all(ent[..., 0] == 1.0) and np.all(ent[..., 1] == 0.0)


@pytest.mark.parametrize("alpha,beta", [(2.0, 2.0), (3.0, 1.0), (float("nan"), 1.0), (0.0, float("inf"))])
def test_fi_ramp_validation(alpha, beta):
    need = ctypes.c_size_t(0)
    assert jl.lib.jl_fi_table(100, 10, 128, 1e4, alpha, beta, None, 0, ctypes.byref(need), None) == jl.JL_EINVAL
    assert jl.lib.jl_fi_table_fill_host(100, 10, 128, 1e4, alpha, beta, FAKE, 1 << 20) == jl.JL_EINVAL
    assert _prefill_fi(alpha=alpha, beta=beta) == jl.JL_EINVAL
    assert _decode_fi(alpha=alpha, beta=beta) == jl.JL_EINVAL


def test_fi_table_size_and_space():
    need = ctypes.c_size_t(0)
    assert jl.lib.jl_fi_table(1000, 100, 128, 1e4, 1.0, 32.0, None, 0, ctypes.byref(need), None) == jl.JL_OK
    assert need.value == 64 + (1024 + 1) * 64 * 8
    assert jl.lib.jl_fi_table(1000, 100, 128, 1e4, 1.0, 32.0, FAKE, need.value - 1, None, None) == jl.JL_ESPACE
    assert jl.lib.jl_fi_table(1000, 0, 128, 1e4, 1.0, 32.0, None, 0, None, None) == jl.JL_EINVAL
    assert jl.lib.jl_fi_table(1000, 100, 96, 1e4, 1.0, 32.0, None, 0, None, None) == jl.JL_EUNSUPPORTED


def _prefill_fi(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=600, Hq=8, Hkv=2,
             D=128, w0=16, wp=64, base=1e4, alpha=1.0, beta=32.0, sc=0.125, table=FAKE, tb=1 << 30, ws=FAKE,
             wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_prefill_fi(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                        a["L"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"], a["base"],
                                        a["alpha"], a["beta"], a["sc"], a["table"], a["tb"], a["ws"], a["wsb"],
                                        None)


def _decode_fi(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=None, i=jl.JL_BF16, o=jl.JL_BF16, B=1, L=600, Lmax=700,
             Hq=8, Hkv=2, D=128, w0=16, wp=64, base=1e4, alpha=1.0, beta=32.0, sc=0.125, ws=FAKE, wsb=1 << 30)
    a.update(over)
    return jl.lib.jl_bifocal_decode_fi(a["q"], a["k"], a["v"], a["out"], a["lse"], a["i"], a["o"], a["B"],
                                       a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], a["w0"], a["wp"], a["base"],
                                       a["alpha"], a["beta"], a["sc"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(table=None), jl.JL_EINVAL), (dict(tb=64), jl.JL_ESPACE), (dict(ws=None), jl.JL_ESPACE),
    (dict(w0=-1), jl.JL_EINVAL), (dict(wp=0), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
    (dict(i=jl.JL_F32, o=jl.JL_BF16), jl.JL_EUNSUPPORTED), (dict(q=FAKE + 4), jl.JL_EINVAL),
])
def test_prefill_fi_validation(over, code):
    assert _prefill_fi(**over) == code


@pytest.mark.parametrize("over,code", [
    (dict(ws=None), jl.JL_EINVAL), (dict(Lmax=599), jl.JL_EINVAL), (dict(wsb=16), jl.JL_ESPACE),
    (dict(i=jl.JL_F32, o=jl.JL_F32), jl.JL_EUNSUPPORTED), (dict(w0=-3), jl.JL_EINVAL),
    (dict(D=32), jl.JL_EUNSUPPORTED), (dict(k=FAKE + 8), jl.JL_EINVAL),
])
def test_decode_fi_validation(over, code):
    assert _decode_fi(**over) == code


@pytest.mark.parametrize("args,code", [
    ((None, FAKE, jl.JL_BF16, 10, 128), jl.JL_EINVAL), ((FAKE, None, jl.JL_BF16, 10, 128), jl.JL_EINVAL),
    ((FAKE, FAKE + 4096, 7, 10, 128), jl.JL_EINVAL), ((FAKE, FAKE + 4096, jl.JL_BF16, 10, 96), jl.JL_EUNSUPPORTED),
    ((FAKE, FAKE + 4096, jl.JL_BF16, -1, 128), jl.JL_EINVAL), ((FAKE + 8, FAKE + 4096, jl.JL_BF16, 10, 128),
                                                              jl.JL_EINVAL),
    ((FAKE, FAKE + 2048, jl.JL_BF16, 10, 128), jl.JL_EINVAL),    # 10 rows of 256 B overlap
    ((FAKE + 2048, FAKE, jl.JL_F32, 5, 128), jl.JL_EINVAL),      # 5 rows of 512 B overlap
])
def test_interleaved_to_half_validation(args, code):
    assert jl.lib.jl_rope_interleaved_to_half(*args, None) == code


def test_call_scratch_is_allocated_on_the_call_stream(monkeypatch):
    """A wrapper that allocates its own workspace does so on the stream its
    kernels run on, so the caching allocator cannot reuse the block for work
    on another stream while those kernels still use it."""
    import types
    from zero_shot_rope_jl_amd import binding
    log = []

    class Ctx:
        def __init__(self, s):
            self.s = s

        def __enter__(self):
            log.append(("enter", self.s))

        def __exit__(self, *a):
            log.append(("exit", self.s))

    fake = types.SimpleNamespace(
        uint8="u8",
        empty=lambda n, dtype, device: log.append(("alloc", n)) or ("buf", n),
        cuda=types.SimpleNamespace(ExternalStream=lambda ptr, device=None: ("ext", ptr),
                                   stream=lambda s: Ctx(s)))
    monkeypatch.setattr(binding, "_torch", lambda: fake)
    assert binding._scratch(64, "cuda:0", 0x1234) == ("buf", 64)
    assert log == [("enter", ("ext", 0x1234)), ("alloc", 64), ("exit", ("ext", 0x1234))]
    log.clear()
    binding._scratch(32, "cuda:0", None)   # torch's current stream: the call runs there too
    assert log == [("alloc", 32)]


def test_decode_noalloc_validation_and_scratch_limit():
    """The no-allocation decode validates like jl_bifocal_decode and refuses,
    before any HIP call, a step whose partials exceed its fixed 16 MiB
    scratch (1024 sequences x 64 heads x one split x 130 floats)."""
    args = lambda **o: dict(dict(B=1, L=600, Lmax=700, Hq=8, Hkv=2, D=128, tab=FAKE), **o)

    def call(a):
        return jl.lib.jl_bifocal_decode_noalloc(FAKE, FAKE, FAKE, FAKE, None, jl.JL_BF16, jl.JL_BF16, a["B"],
                                                a["L"], a["Lmax"], a["Hq"], a["Hkv"], a["D"], 16, 64, 1e4, 0.125,
                                                a["tab"], 1 << 40, None)
    assert call(args(Lmax=599)) == jl.JL_EINVAL
    assert call(args(tab=None)) == jl.JL_EINVAL
    assert call(args(D=96)) == jl.JL_EUNSUPPORTED
    assert call(args(B=1024, L=64, Lmax=64, Hq=64, Hkv=8)) == jl.JL_ESPACE
    assert "scratch" in jl.jl_last_error()


def test_prefill_chunk_workspace_size():
    """Rotated keys [B, Lcap, Hkv, D] bf16 (when G can exceed 1), rounded up to
    256 bytes, then room for the larger of two partial sets: the prefill
    kernels' key splits (a chunk whose query tiles give under 128 workgroups
    is split into as many parts as keep it within 256 workgroups, one per
    compute unit, >= 4 key tiles each, <= 64), and the decode kernels'
    splits for chunks of at most 64 (position, query head) columns per KV
    head ([B, Lq, Hq, n_split, D + 2] fp32, about 256 workgroups)."""
    up = lambda x: (x + 255) // 256 * 256

    def need_rows(lq_max, keys, R=4, Hkv=8):
        best = 0
        for lq in range(1, lq_max + 1):
            wgs = -(-lq // (256 // R)) * Hkv
            tiles = -(-keys // 128)
            if wgs >= 128 or tiles < 8:
                continue
            s = min(256 // wgs, tiles // 4, 64)
            best = max(best, s * lq if s > 1 else 0)
        return best

    def dec_bytes(lq_max, keys, Hq=32, Hkv=8, D=128, B=1):
        # column groups of 16: 1, 2 or 4, each group count with its longest chunk.
        # One group: the split kernel, up to 4 KV heads per workgroup, 32-key
        # steps; 2 or 4: one KV head per workgroup, 64-key stages; ~256 workgroups
        R, best = Hq // Hkv, 0
        for ng in (1, 2, 4):
            lq = min(lq_max, 16 * ng // R)
            cols = lq * R
            if lq < 1 or (1 if cols <= 16 else 2 if cols <= 32 else 4) != ng or B * lq > 65535:
                continue
            if ng == 1:
                groups = B * Hkv // min(4, Hkv)
                n_split = min(256 // groups if groups < 256 else 1, min(-(-keys // 32), 256))
            else:
                groups = B * Hkv
                n_split = min(-(-256 // groups) if groups < 256 else 1, -(-keys // 64))
            best = max(best, B * lq * Hq * n_split * (D + 2) * 4)
        return best

    # 131072-row cache, 16-token chunk, 32/8 heads: 8 workgroups -> 32 prefill
    # splits, against 32 decode splits of 16 x 32 columns (4 groups, one KV head
    # per workgroup): the prefill partials (132 floats a row) are the larger
    assert dec_bytes(16, 131072) == 16 * 32 * 32 * 130 * 4
    n = jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 16, 131072, 32, 8, 128, 32768)
    assert n == up(131072 * 8 * 128 * 2) + 32 * 16 * 32 * 132 * 4
    # a 4096-token chunk fills 512 workgroups and is not split, but a workspace for
    # chunks of up to 4096 tokens has room for the splits of shorter ones: the
    # largest need is 32 splits x 64 rows (8 workgroups; 960 tokens need 2 x 960)
    n = jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 4096, 131072, 32, 8, 128, 32768)
    assert need_rows(4096, 131072) == 32 * 64
    assert n == up(131072 * 8 * 128 * 2) + 32 * 64 * 32 * 132 * 4
    # up to 256 tokens: the same largest need (192 tokens need 10 x 192, 256 tokens
    # 8 x 256)
    assert need_rows(256, 131072) == 32 * 64
    n = jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 256, 131072, 32, 8, 128, 32768)
    assert n == up(131072 * 8 * 128 * 2) + 32 * 64 * 32 * 132 * 4
    # the size never shrinks as the chunk bound grows
    sizes = [jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, lq, 1500, 8, 2, 128, 400) for lq in range(1, 300)]
    assert all(a <= b for a, b in zip(sizes, sizes[1:]))
    # a cache within the pretrained window needs no rotated keys; 9 key tiles give
    # 2 prefill splits, but the decode kernels' 18 splits (64-key stages) of 16 x 32
    # columns are larger
    assert dec_bytes(16, 1100) == 16 * 32 * 18 * 130 * 4
    assert jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 16, 1100, 32, 8, 128, 32768) == \
        16 * 32 * 18 * 130 * 4
    # fewer than 8 key tiles: no prefill split; a 4-token chunk (16 columns, 4 heads
    # per workgroup, 2 groups of them -> 128 splits, 28 at 896 keys)
    assert jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 4, 896, 32, 8, 128, 32768) == \
        4 * 32 * 28 * 130 * 4 == dec_bytes(4, 896)
    # B * Lq above 65535 would overflow the decode combine's grid, so 1024 sequences
    # of 64 tokens stay on the prefill kernels (unsplit at 8192 workgroups): the
    # room is for chunks of up to 32 tokens on the decode kernels (one split each)
    assert jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1024, 64, 896, 8, 8, 128, 32768) == \
        1024 * 32 * 8 * 1 * 130 * 4 == dec_bytes(32, 896, Hq=8, Hkv=8, B=1024)
    # fp32 inputs: the generic kernel rotates its keys itself and does not split
    assert jl.jl_bifocal_prefill_chunk_workspace(jl.JL_F32, 1, 16, 131072, 32, 8, 128, 32768) == 0
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, 1, 17, 16, 32, 8, 128, 32768)


def test_prefill_chunk_workspace_is_monotone_over_random_shapes():
    """The room a chunk workspace sizes for (Lq, Lcap) must cover every call
    with a chunk of at most Lq tokens over at most Lcap keys: the size never
    shrinks as either bound grows, over seeded random shapes (bf16, both
    routes, split and unsplit plans)."""
    rng = np.random.Generator(np.random.PCG64(99))
    for _ in range(24):
        Hkv = int(rng.choice([1, 2, 4, 8]))
        Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
        B, D, w_pre = int(rng.integers(1, 4)), int(rng.choice([64, 128])), int(rng.integers(16, 5000))
        ws = lambda lq, cap: jl.jl_bifocal_prefill_chunk_workspace(jl.JL_BF16, B, lq, cap, Hq, Hkv, D, w_pre)
        caps = sorted(set(int(c) for c in rng.integers(1, 40000, 6)))
        lqs = sorted(set(int(x) for x in rng.integers(1, 1200, 6)))
        for cap in caps:
            sizes = [ws(lq, cap) for lq in lqs if lq <= cap]
            assert all(a <= b for a, b in zip(sizes, sizes[1:])), (B, Hq, Hkv, D, w_pre, cap)
        for lq in lqs:
            sizes = [ws(lq, cap) for cap in caps if cap >= lq]
            assert all(a <= b for a, b in zip(sizes, sizes[1:])), (B, Hq, Hkv, D, w_pre, lq)
