"""Pins for the float64 oracle against what the Jet-Long pages and the
mathematics fix.  CPU only.

Each pin reaches the answer by a route other than the oracle's own code:
transcribed schedule values, a minimality characterisation of G, complex
exponentials for RoPE, scalar Python loops, a library attention routine,
and exact identities stated on the pages.
"""
import cmath
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import jetlong_oracle as jo
import synth_inputs as si

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers
def rope_complex(x, pos, base):
    """RoPE from scratch: channel pair (i, i + D/2) as the complex number
    x_i + j x_{i+D/2}, multiplied by exp(j * pos * base^(-2i/D))."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    h = D // 2
    i = np.arange(h)
    th = np.array([base ** (-2.0 * ii / D) for ii in i])
    z = x[..., :h] + 1j * x[..., h:]
    z = z * np.exp(1j * np.asarray(pos, dtype=np.float64)[..., None] * th)
    return np.concatenate([z.real, z.imag], axis=-1)


def brute_force(q, k, v, w0, w_pre, base, scale, interleaved=False):
    """Scalar loops: remote scores rebuild RoPE(x, f(p)) by undoing the
    stored phase p and applying f(p) (two rotations per vector, from cos/sin
    of p*theta and f(p)*theta), instead of the oracle's single offset.
    Frequency i rotates the channel pair (i, i + D/2), or (2i, 2i + 1) when
    ``interleaved``."""
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    R = Hq // Hkv
    h2 = D // 2
    G = max(1, -(-L // w_pre))        # written independently of the oracle
    th = [base ** (-2.0 * i / D) for i in range(h2)]

    def realias(vec, p):
        fp = p // G
        out = [0.0] * D
        for i in range(h2):
            a, c = (2 * i, 2 * i + 1) if interleaved else (i, i + h2)
            z = complex(vec[a], vec[c])
            z = z * cmath.exp(-1j * p * th[i])      # undo stored phase
            z = z * cmath.exp(1j * fp * th[i])      # aliased phase
            out[a], out[c] = z.real, z.imag
        return out

    out = np.zeros((B, L, Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // R
            for qi in range(L):
                qv = list(q[b, qi, h])
                qr = realias(qv, qi)
                sc = []
                for ki in range(qi + 1):
                    kv = list(k[b, ki, g])
                    if qi - ki <= w0:
                        s = sum(a * c for a, c in zip(qv, kv))
                    else:
                        s = sum(a * c for a, c in zip(qr, realias(kv, ki)))
                    sc.append(s * scale)
                m = max(sc)
                e = [math.exp(s - m) for s in sc]
                tot = sum(e)
                for d in range(D):
                    out[b, qi, h, d] = sum(e[ki] * v[b, ki, g, d] for ki in range(qi + 1)) / tot
    return out


def rand_qkv(seed, B, L, Hq, Hkv, D):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, L, Hq, D)), rng.standard_normal((B, L, Hkv, D)),
            rng.standard_normal((B, L, Hkv, D)))


# ------------------------------------------------------------ I3 schedule
def test_schedule_values_from_pages():
    with open(os.path.join(GOLDEN, "schedule_examples.json")) as fh:
        ex = json.load(fh)["examples"]
    assert len(ex) >= 5
    for e in ex:
        assert oracle.group_size(e["L"], e["w_pretrained"]) == e["G"], e["cite"]


@pytest.mark.parametrize("w_pre", [1, 2, 3, 7, 64, 1000])
def test_schedule_is_minimal_integer_compression(w_pre):
    # §3.1: G is the smallest integer grouping that keeps every aliased
    # position 0..L-1 inside the pretrained range [0, w_pre).
    for L in list(range(1, 3 * w_pre + 5)) + [50 * w_pre + 1]:
        G = oracle.group_size(L, w_pre)
        assert (L - 1) // G <= w_pre - 1
        smallest = next(g for g in range(1, L + 2) if (L - 1) // g <= w_pre - 1)
        assert G == smallest
        if L <= w_pre:
            assert G == 1
            assert np.array_equal(oracle.alias_position(np.arange(L), G), np.arange(L))


def test_schedule_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.group_size(0, 10)
    with pytest.raises(ValueError):
        oracle.group_size(10, 0)


def test_alias_and_offset():
    p = np.arange(0, 40)
    G = 3
    assert np.array_equal(oracle.alias_position(p, G), np.array([x // 3 for x in range(40)]))
    assert np.array_equal(oracle.correction_offset(p, G), np.array([x // 3 - x for x in range(40)]))


# ---------------------------------------------- RoPE and I5 correction
def test_inv_freq_values():
    th = oracle.inv_freq(8, 10000.0)
    assert th[0] == 1.0
    np.testing.assert_allclose(th, [1.0, 0.1, 0.01, 0.001], rtol=1e-15)


def test_rope_rotate_matches_complex_exponential():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 16))
    pos = rng.integers(-200000, 200000, size=(5, 3))
    np.testing.assert_allclose(oracle.rope_rotate(x, pos, 1e6), rope_complex(x, pos, 1e6),
                               atol=1e-11, rtol=0)


@pytest.mark.parametrize("G", [1, 2, 3, 5])
def test_correction_recovers_aliased_phase(G):
    # §3.2 Eq. (5): rotating RoPE(x, p) by f(p) - p gives RoPE(x, f(p)).
    rng = np.random.default_rng(10 + G)
    L, D = 300, 32
    x = rng.standard_normal((1, L, 2, D))
    p = np.arange(L)
    stored = rope_complex(x, p[None, :, None], 1e4)
    got = oracle.remote_view(stored, p, G, 1e4)
    want = rope_complex(x, (p // G)[None, :, None], 1e4)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_correction_precise_at_long_positions():
    # Offsets up to ~1.05e5 (G = 5 at 131K): the float64 angle stays accurate.
    rng = np.random.default_rng(11)
    D = 128
    p = np.array([131327, 131072, 98305, 65535])
    x = rng.standard_normal((1, 4, 1, D))
    stored = rope_complex(x, p[None, :, None], 1e6)
    got = oracle.remote_view(stored, p, 5, 1e6)
    want = rope_complex(x, (p // 5)[None, :, None], 1e6)
    np.testing.assert_allclose(got, want, atol=1e-9, rtol=0)


# ---------------------------------------------------------- I4 brute force
CASES = [  # (L, w_pre, w0, D, Hq, Hkv)
    (1, 1, 0, 2, 1, 1), (5, 1, 0, 2, 2, 1), (9, 2, 1, 4, 2, 2), (12, 3, 2, 4, 2, 1),
    (17, 4, 0, 8, 1, 1), (23, 5, 3, 8, 2, 1), (31, 9, 6, 4, 4, 2), (40, 7, 40, 8, 2, 2),
    (40, 6, 39, 4, 2, 1), (40, 40, 5, 4, 2, 1), (33, 8, 7, 8, 2, 2), (26, 2, 12, 2, 1, 1),
]


@pytest.mark.parametrize("case", CASES)
def test_bruteforce_matches_oracle(case):
    L, w_pre, w0, D, Hq, Hkv = case
    q, k, v = rand_qkv(hash(case) % 2**31, 1, L, Hq, Hkv, D)
    # large-ish entries so that the remote/local difference matters
    q *= 1.5
    k *= 1.5
    scale = 1.0 / math.sqrt(D)
    want = brute_force(q, k, v, w0, w_pre, 1e4, scale)
    got, _ = oracle.bifocal_attention(q, k, v, w0, w_pre, 1e4, scale, block=7)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_bruteforce_sweep_small():
    # every w0 for a few (L, w_pre) shapes, D = 2 and 4, GQA 1 and 2
    for (L, w_pre, D, Hq, Hkv) in [(11, 3, 2, 1, 1), (14, 4, 4, 2, 1), (9, 2, 4, 2, 2)]:
        q, k, v = rand_qkv(L * 100 + w_pre, 1, L, Hq, Hkv, D)
        q *= 2.0
        k *= 2.0
        for w0 in range(0, L + 1):
            want = brute_force(q, k, v, w0, w_pre, 100.0, 0.5)
            got, _ = oracle.bifocal_attention(q, k, v, w0, w_pre, 100.0, 0.5, block=4)
            np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)


def test_interleaved_pairing_is_a_channel_permutation():
    # A model whose RoPE pairs channels (2i, 2i+1) uses the rotate-half path
    # with q and k channels permuted so that pair i lands on (i, i + D/2):
    # the scores, hence the output, do not change (v is not permuted).
    L, w_pre, w0, D, Hq, Hkv = 23, 5, 3, 8, 2, 1
    q, k, v = rand_qkv(77, 1, L, Hq, Hkv, D)
    q *= 1.5
    k *= 1.5
    want = brute_force(q, k, v, w0, w_pre, 1e4, 0.4, interleaved=True)
    perm = [2 * j for j in range(D // 2)] + [2 * j + 1 for j in range(D // 2)]
    got, _ = oracle.bifocal_attention(q[..., perm], k[..., perm], v, w0, w_pre, 1e4, 0.4, block=5)
    np.testing.assert_allclose(got, want, atol=1e-12, rtol=0)
    # without the permutation the two conventions differ
    other, _ = oracle.bifocal_attention(q, k, v, w0, w_pre, 1e4, 0.4, block=5)
    assert np.abs(other - want).max() > 1e-3


# ------------------------------------------------------ I1 exact identity
@pytest.mark.parametrize("L,w_pre,w0", [(64, 64, 8), (50, 1000, 0), (64, 16, 63), (64, 16, 200)])
def test_identity_regime_is_plain_attention_bitwise(L, w_pre, w0):
    # L <= w_pre (G = 1) or w0 >= L-1: every pair scores with the stored
    # vectors, so the output must equal plain causal attention exactly.
    q, k, v = rand_qkv(L + w_pre + w0, 2, L, 4, 2, 16)
    a, la = oracle.bifocal_attention(q, k, v, w0, w_pre, 1e4, 0.25)
    b, lb = oracle.plain_causal_attention(q, k, v, 0.25)
    assert np.array_equal(a, b)
    assert np.array_equal(la, lb)


def test_identity_regime_ignores_w0():
    q, k, v = rand_qkv(5, 1, 48, 2, 1, 8)
    outs = [oracle.bifocal_attention(q, k, v, w0, 48, 1e4, 0.3)[0] for w0 in (0, 1, 17, 47)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# -------------------------------------------------- I2 textbook routine
def test_plain_matches_torch_sdpa_float64():
    q, k, v = rand_qkv(21, 2, 70, 6, 3, 16)
    scale = 0.3
    got, lse = oracle.plain_causal_attention(q, k, v, scale, block=16)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(2, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, scale=scale)
    np.testing.assert_allclose(got, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12, rtol=0)
    # LSE against torch.logsumexp of the masked score matrix
    S = torch.einsum("bhqd,bhkd->bhqk", tq, tk) * scale
    S = S.masked_fill(torch.ones(70, 70, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(S, dim=-1).numpy(), atol=1e-12, rtol=0)


# --------------------------------------------------- I6 three-pass merge
@pytest.mark.parametrize("L,w_pre,w0", [(40, 8, 5), (64, 16, 0), (33, 4, 31), (50, 10, 12)])
def test_inclusion_exclusion_equals_dense(L, w_pre, w0):
    q, k, v = rand_qkv(L * w0 + 1, 1, L, 4, 2, 8)
    dense, _ = oracle.bifocal_attention(q, k, v, w0, w_pre, 1e4, 0.35)
    ie = oracle.inclusion_exclusion_attention(q, k, v, w0, w_pre, 1e4, 0.35)
    np.testing.assert_allclose(ie, dense, atol=1e-10, rtol=0)


# ------------------------------------------------------ I7 special cases
def test_single_token_and_first_row():
    q, k, v = rand_qkv(7, 1, 1, 2, 1, 8)
    o, lse = oracle.bifocal_attention(q, k, v, 0, 1, 1e4, 0.5)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]) and np.array_equal(o[0, 0, 1], v[0, 0, 0])
    q, k, v = rand_qkv(8, 1, 30, 2, 1, 8)
    o, _ = oracle.bifocal_attention(q, k, v, 3, 4, 1e4, 0.5)
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0])
    s00 = 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])
    _, lse = oracle.bifocal_attention(q, k, v, 3, 4, 1e4, 0.5, rows=[0])
    assert abs(lse[0, 0, 0] - s00) < 1e-14


def test_pretrained_window_one_makes_far_keys_position_free():
    # w_pre = 1 gives G = L and f = 0: far scores use the un-rotated vectors.
    L, D = 20, 8
    rng = np.random.default_rng(4)
    x_q = rng.standard_normal((1, L, 1, D))
    x_k = rng.standard_normal((1, L, 1, D))
    v = rng.standard_normal((1, L, 1, D))
    p = np.arange(L)[None, :, None]
    q = rope_complex(x_q, p, 1e4)
    k = rope_complex(x_k, p, 1e4)
    w0 = 2
    o, _ = oracle.bifocal_attention(q, k, v, w0, 1, 1e4, 0.4)
    for qi in (5, 19):
        sc = []
        for ki in range(qi + 1):
            s = q[0, qi, 0] @ k[0, ki, 0] if qi - ki <= w0 else x_q[0, qi, 0] @ x_k[0, ki, 0]
            sc.append(0.4 * s)
        e = np.exp(np.array(sc) - max(sc))
        want = (e[:, None] * v[0, :qi + 1, 0]).sum(0) / e.sum()
        np.testing.assert_allclose(o[0, qi, 0], want, atol=1e-12, rtol=0)


def test_window_zero_keeps_only_the_diagonal_local():
    # w0 = 0: only the self pair keeps its true RoPE phases (Table 16 caption).
    L, D, G_wpre = 16, 4, 4
    q, k, v = rand_qkv(9, 1, L, 1, 1, D)
    o, _ = oracle.bifocal_attention(q, k, v, 0, G_wpre, 1e4, 1.0)
    want = brute_force(q, k, v, 0, G_wpre, 1e4, 1.0)
    np.testing.assert_allclose(o, want, atol=1e-12)
    # changing an off-diagonal local pair's phase handling would move row 3;
    # check that w0 = 0 and w0 = 1 really differ there
    o1, _ = oracle.bifocal_attention(q, k, v, 1, G_wpre, 1e4, 1.0)
    assert np.abs(o1[0, 3] - o[0, 3]).max() > 1e-6


# ----------------------------------------- I8 decode/prefill consistency
@pytest.mark.parametrize("L,w_pre,w0", [(37, 8, 4), (64, 64, 3), (90, 7, 20)])
def test_decode_equals_last_prefill_row(L, w_pre, w0):
    q, k, v = rand_qkv(L, 2, L, 4, 2, 8)
    full, lse = oracle.bifocal_attention(q, k, v, w0, w_pre, 1e4, 0.4)
    kc = np.concatenate([k, np.full((2, 5, 2, 8), 1e9)], axis=1)  # rows >= L must be ignored
    vc = np.concatenate([v, np.full((2, 5, 2, 8), 1e9)], axis=1)
    o, ls = oracle.decode_attention(q[:, L - 1], kc, vc, L, w0, w_pre, 1e4, 0.4)
    np.testing.assert_allclose(o, full[:, L - 1], atol=1e-12, rtol=0)
    np.testing.assert_allclose(ls, lse[:, :, L - 1], atol=1e-12, rtol=0)


# ------------------------------------------------------ I9 convexity
def test_convexity_and_unit_weights():
    q, k, v = rand_qkv(12, 1, 80, 4, 2, 8)
    q *= 3
    o, _ = oracle.bifocal_attention(q, k, v, 10, 16, 1e4, 0.5)
    for h in range(4):
        g = h // 2
        for qi in range(80):
            lo = v[0, :qi + 1, g].min(0) - 1e-12
            hi = v[0, :qi + 1, g].max(0) + 1e-12
            assert np.all(o[0, qi, h] >= lo) and np.all(o[0, qi, h] <= hi)
    ones = np.ones_like(v)
    o1, _ = oracle.bifocal_attention(q, k, ones, 10, 16, 1e4, 0.5)
    np.testing.assert_allclose(o1, 1.0, atol=1e-14)


# ------------------------------------------------ sampled rows = full rows
def test_row_subset_matches_full_evaluation():
    q, k, v = rand_qkv(13, 1, 100, 2, 1, 8)
    full, lf = oracle.bifocal_attention(q, k, v, 9, 30, 1e4, 0.4)
    rows = np.array([0, 1, 9, 10, 11, 29, 30, 31, 59, 60, 99])
    sub, ls = oracle.bifocal_attention(q, k, v, 9, 30, 1e4, 0.4, rows=rows)
    np.testing.assert_allclose(sub, full[:, rows], atol=1e-12, rtol=0)
    np.testing.assert_allclose(ls, lf[:, :, rows], atol=1e-12, rtol=0)


# --------------------------------------------------- generator rounding
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -3.0078125, 0.0], np.float32)])
    bits = si.bf16_bits_from_f32(x)
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, tb)
    assert np.array_equal(si.f32_from_bf16_bits(bits), torch.from_numpy(tb.view(np.int16)).view(
        torch.bfloat16).float().numpy())
