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
                           "jl_rope_interleaved_to_half"])
    for s in syms:
        assert hasattr(jl.lib, s), s
    assert jl.jl_version() == 8


def test_schedule_golden_and_table_size():
    with open(os.path.join(ROOT, "tests", "golden", "schedule_examples.json")) as fh:
        for e in json.load(fh)["examples"]:
            G, need = jl.jl_schedule(e["L"], e["w_pretrained"], 128, 1e6)
            assert G == e["G"], e["cite"]
            assert need == 64 + e["L"] * 64 * 8


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
    # bf16 with G = ceil(L / w_pretrained) > 1: the keys in their remote view, B*L*Hkv*D bf16
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 1, 131072, 8, 128, 32768) == 131072 * 8 * 128 * 2
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 2, 300, 2, 64, 256) == 2 * 300 * 2 * 64 * 2
    # G == 1 (every pair local) or fp32 inputs: none
    assert jl.jl_bifocal_prefill_workspace(jl.JL_BF16, 1, 4096, 8, 128, 4096) == 0
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
# 256*2*128*2 B, then three fp32 outputs of 256*4*128*4 B and three fp32
# log-sum-exps of 4*256*4 B, every part a multiple of 256 B already
UNFUSED_WS = 256 * 2 * 128 * 2 + 3 * 256 * 4 * 128 * 4 + 3 * 4 * 256 * 4


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
                                           None)


@pytest.mark.parametrize("over,code", [
    (dict(Lq=0), jl.JL_EINVAL), (dict(Lq=601), jl.JL_EINVAL), (dict(Lmax=599), jl.JL_EINVAL),
    (dict(L=0), jl.JL_EINVAL), (dict(q=None), jl.JL_EINVAL), (dict(out=FAKE + 2), jl.JL_EINVAL),
    (dict(D=96), jl.JL_EUNSUPPORTED), (dict(Hq=32, Hkv=2), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE),
    (dict(ws=None), jl.JL_ESPACE), (dict(wsb=600 * 2 * 128 * 2 - 1), jl.JL_ESPACE),
    (dict(i=jl.JL_F32, o=jl.JL_BF16), jl.JL_EUNSUPPORTED), (dict(Lmax=(1 << 30) + 1), jl.JL_EINVAL),
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
                                                 a["table"], a["tb"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("over,code", [
    (dict(bt=None), jl.JL_EINVAL), (dict(bt=FAKE + 2), jl.JL_EINVAL), (dict(ps=64), jl.JL_EINVAL),
    (dict(ps=192), jl.JL_EINVAL), (dict(ps=0), jl.JL_EINVAL), (dict(npg=0), jl.JL_EINVAL),
    (dict(mp=4), jl.JL_EINVAL), (dict(mp=0), jl.JL_EINVAL), (dict(Lq=0), jl.JL_EINVAL),
    (dict(Lq=601), jl.JL_EINVAL), (dict(q=None), jl.JL_EINVAL), (dict(D=96), jl.JL_EUNSUPPORTED),
    (dict(i=jl.JL_F32, o=jl.JL_F32), jl.JL_EUNSUPPORTED), (dict(tb=100), jl.JL_ESPACE),
    (dict(ws=None), jl.JL_ESPACE), (dict(wsb=600 * 2 * 128 * 2 - 1), jl.JL_ESPACE),
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


def test_decode_workspace_size():
    assert jl.jl_bifocal_decode_workspace(1, 32, 128, 131328) == 32 * 256 * 130 * 4
    assert jl.jl_bifocal_decode_workspace(1, 32, 128, 1000) == 32 * 32 * 130 * 4
    assert jl.jl_bifocal_decode_workspace(2, 4, 64, 1) == 2 * 4 * 1 * 66 * 4
    with pytest.raises(jl.JetLongError):
        jl.jl_bifocal_decode_workspace(1, 4, 96, 10)


@pytest.mark.parametrize("D,base,L", [(64, 1e4, 512), (128, 1e6, 131328), (128, 5e5, 1)])
def test_host_table_matches_numpy_float64(D, base, L):
    buf = jl.jl_table_fill_host(L, D, base)
    hdr = buf[:64]
    assert hdr[:4].view(np.uint32)[0] == 0x324C544A
    assert hdr[4:8].view(np.int32)[0] == D
    assert hdr[8:16].view(np.int64)[0] == L
    assert hdr[16:24].view(np.float64)[0] == base
    ent = buf[64:].view(np.float32).reshape(L, D // 2, 2)
    theta = base ** (-(2.0 * np.arange(D // 2)) / D)          # independent float64 definition
    ang = np.arange(L, dtype=np.float64)[:, None] * theta[None, :]
    want = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    # one fp32 ulp of rounding plus the float64 angle error (|n * d(theta)| < 1e-10)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ent.astype(np.float64) - want) <= ulp + 1e-10)


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
    ent = buf[64:].view(np.float32).reshape(L, D // 2, 2)
    phi = oracle.inv_freq(D, base) - oracle.fi_inv_freq(D, base, L, w_pre, alpha, beta)
    ang = np.arange(L, dtype=np.float64)[:, None] * phi[None, :]
    want = np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)
    ulp = np.spacing(np.abs(want).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(ent.astype(np.float64) - want) <= ulp + 1e-10)
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
    assert need.value == 64 + 1000 * 64 * 8
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
