"""Pins for the oracle's frequency-interpolation remote view (Jet-Long §4.7
ablation, with the continuous ratio s = max(1, L / w_pretrained) of §3.1).
CPU only.

The brute force here starts from raw vectors x, builds the stored vectors
RoPE(x, p) and the remote scores from x rotated straight to the
interpolated phases, in scalar loops with complex exponentials and with each
pair's frequency chosen by explicit cases, instead of the oracle's single
correction rotation of the stored vector.
"""
import cmath
import math

import numpy as np
import pytest

from oracle import jetlong_oracle as jo


def _thetas(D, base):
    return [base ** (-2.0 * i / D) for i in range(D // 2)]


def _interp_freq(D, base, L, w_pre, alpha, beta):
    """theta'_i pair by pair: kept above beta turns per window, divided by s
    below alpha, a linear blend between."""
    s = max(1.0, L / w_pre)
    out = []
    for th in _thetas(D, base):
        turns = w_pre / (2.0 * math.pi / th)
        if turns > beta:
            out.append(th)
        elif turns < alpha:
            out.append(th / s)
        else:
            g = (turns - alpha) / (beta - alpha)
            out.append(g * th + (1.0 - g) * th / s)
    return out


def _rot(vec, pos, freqs):
    D = len(vec)
    h = D // 2
    out = [0.0] * D
    for i in range(h):
        z = complex(vec[i], vec[i + h]) * cmath.exp(1j * pos * freqs[i])
        out[i], out[i + h] = z.real, z.imag
    return out


def _stored(x, base):
    """RoPE(x, p) for raw x [B, L, H, D] at positions 0..L-1."""
    B, L, H, D = x.shape
    th = _thetas(D, base)
    u = np.empty_like(x)
    for b in range(B):
        for p in range(L):
            for h in range(H):
                u[b, p, h] = _rot(list(x[b, p, h]), p, th)
    return u


def _brute(xq, xk, v, w0, w_pre, base, alpha, beta, scale):
    """Attention from raw vectors: local pairs score RoPE(x, p) vectors,
    remote pairs the raw vectors rotated to p * theta'_i."""
    B, L, Hq, D = xq.shape
    Hkv = xk.shape[2]
    R = Hq // Hkv
    th = _thetas(D, base)
    thp = _interp_freq(D, base, L, w_pre, alpha, beta)
    out = np.zeros((B, L, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // R
            for qi in range(L):
                ql, qr = _rot(list(xq[b, qi, h]), qi, th), _rot(list(xq[b, qi, h]), qi, thp)
                sc = []
                for ki in range(qi + 1):
                    if qi - ki <= w0:
                        kv = _rot(list(xk[b, ki, g]), ki, th)
                        sc.append(sum(a * c for a, c in zip(ql, kv)) * scale)
                    else:
                        kv = _rot(list(xk[b, ki, g]), ki, thp)
                        sc.append(sum(a * c for a, c in zip(qr, kv)) * scale)
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, qi, h, d] = sum(e[k] * v[b, k, g, d] for k in range(qi + 1)) / tot
    return out


def _raw(seed, B, L, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    return (1.5 * rng.standard_normal((B, L, Hq, D)), 1.5 * rng.standard_normal((B, L, Hkv, D)),
            rng.standard_normal((B, L, Hkv, D)))


# D = 16, base 1e4, w_pre 6: pair i turns 6 * 10^(-i/2) / (2 pi) times per
# window, i.e. 0.95, 0.30, 0.095, ...  The ramps below put pairs on each side.
RAMPS = [
    (0.05, 0.5),     # pair 0 kept, pair 1 on the ramp, pair 2 on the ramp, the rest divided by s
    (-2.0, -1.0),    # every pair kept
    (50.0, 100.0),   # every pair divided by s: position interpolation
    (0.2, 2.0),      # pairs 0 and 1 on the ramp
]


@pytest.mark.parametrize("ramp", RAMPS)
@pytest.mark.parametrize("L,w0", [(17, 3), (23, 0)])
def test_fi_matches_brute_force_from_raw_vectors(ramp, L, w0):
    alpha, beta = ramp
    B, Hq, Hkv, D, w_pre, base = 1, 2, 1, 16, 6, 1e4
    xq, xk, v = _raw(L + w0, B, L, Hq, Hkv, D)
    q, k = _stored(xq, base), _stored(xk, base)
    want = _brute(xq, xk, v, w0, w_pre, base, alpha, beta, 1 / math.sqrt(D))
    got, _ = jo.bifocal_attention_fi(q, k, v, w0, w_pre, base, alpha, beta, 1 / math.sqrt(D), block=7)
    assert np.allclose(got, want, atol=1e-11, rtol=0)


def test_fi_within_the_pretrained_window_is_plain_attention():
    """s = 1: the interpolated frequencies are the stored ones, exactly."""
    q, k, v = _raw(3, 1, 40, 4, 2, 16)
    for L in (40, 39):
        got, gl = jo.bifocal_attention_fi(q[:, :L], k[:, :L], v[:, :L], 2, 40, 1e4, 1.0, 32.0, 0.25)
        want, wl = jo.plain_causal_attention(q[:, :L], k[:, :L], v[:, :L], 0.25)
        assert np.array_equal(got, want) and np.array_equal(gl, wl)


def test_fi_every_pair_kept_is_plain_attention():
    q, k, v = _raw(4, 1, 50, 4, 2, 16)
    got, _ = jo.bifocal_attention_fi(q, k, v, 5, 8, 1e4, -2.0, -1.0, 0.25)
    want, _ = jo.plain_causal_attention(q, k, v, 0.25)
    assert np.array_equal(got, want)


def test_fi_window_covering_every_pair_is_plain_attention():
    q, k, v = _raw(5, 1, 30, 4, 2, 16)
    got, _ = jo.bifocal_attention_fi(q, k, v, 29, 4, 1e4, 1.0, 32.0, 0.25)
    want, _ = jo.plain_causal_attention(q, k, v, 0.25)
    assert np.array_equal(got, want)


def test_fi_scale_is_continuous():
    """§3.1: s = max(1, L / w_pretrained), not rounded up like G."""
    assert jo.fi_scale(100, 100) == 1.0 and jo.fi_scale(50, 100) == 1.0
    assert jo.fi_scale(150, 100) == 1.5 and jo.fi_scale(131072, 32768) == 4.0
    assert jo.fi_scale(131073, 32768) == pytest.approx(4.0000305, rel=1e-7)


def test_fi_decode_is_the_last_prefill_row():
    q, k, v = _raw(6, 2, 45, 4, 2, 16)
    L = 45
    o, l = jo.decode_attention_fi(q[:, L - 1], k, v, L, 4, 10, 1e4, 0.05, 0.5, 0.25)
    po, pl = jo.bifocal_attention_fi(q, k, v, 4, 10, 1e4, 0.05, 0.5, 0.25, rows=[L - 1])
    assert np.allclose(o, po[:, 0], atol=1e-13, rtol=0) and np.allclose(l, pl[:, :, 0], atol=1e-13, rtol=0)


# ---------------------------------------------------------------- mutations
def _fi_pins_fail() -> bool:
    for ramp in RAMPS:
        for L, w0 in [(17, 3)]:
            alpha, beta = ramp
            xq, xk, v = _raw(L + w0, 1, L, 2, 1, 16)
            q, k = _stored(xq, 1e4), _stored(xk, 1e4)
            want = _brute(xq, xk, v, w0, 6, 1e4, alpha, beta, 0.25)
            got, _ = jo.bifocal_attention_fi(q, k, v, w0, 6, 1e4, alpha, beta, 0.25)
            if not np.allclose(got, want, atol=1e-11, rtol=0):
                return True
    return False


def _mut_sign(mp):
    orig = jo.fi_inv_freq
    mp.setattr(jo, "fi_inv_freq", lambda D, b, L, w, a, c: 2 * jo.inv_freq(D, b) - orig(D, b, L, w, a, c))


def _mut_ramp_reversed(mp):
    orig = jo.fi_ramp
    mp.setattr(jo, "fi_ramp", lambda D, b, w, a, c: 1.0 - orig(D, b, w, a, c))


def _mut_scale_rounded_up(mp):
    mp.setattr(jo, "fi_scale", lambda L, w: float(max(1, -(-L // w))))


def _mut_ramp_over_wavelength(mp):
    mp.setattr(jo, "fi_ramp", lambda D, b, w, a, c: np.clip(
        (2 * np.pi / jo.inv_freq(D, b) / w - a) / (c - a), 0.0, 1.0))


def _mut_scale_multiplies(mp):
    orig = jo.fi_scale
    mp.setattr(jo, "fi_scale", lambda L, w: 1.0 / orig(L, w))


@pytest.mark.parametrize("mut", [_mut_sign, _mut_ramp_reversed, _mut_scale_rounded_up, _mut_ramp_over_wavelength,
                                 _mut_scale_multiplies])
def test_fi_pins_catch_planted_mistake(mut, monkeypatch):
    assert not _fi_pins_fail()
    mut(monkeypatch)
    assert _fi_pins_fail()
