"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that the pins in test_oracle_pins catch every one of them."""
import json
import math
import os

import numpy as np
import pytest

from oracle import jetlong_oracle as jo
import test_oracle_pins as pins


def _pins_fail() -> bool:
    """Run a compact set of the pins; True if any of them fails."""
    with open(os.path.join(pins.GOLDEN, "schedule_examples.json")) as fh:
        for e in json.load(fh)["examples"]:
            if jo.group_size(e["L"], e["w_pretrained"]) != e["G"]:
                return True
    for case in [(23, 5, 3, 8, 2, 1), (31, 9, 6, 4, 4, 2), (12, 3, 2, 4, 2, 1)]:
        L, w_pre, w0, D, Hq, Hkv = case
        q, k, v = pins.rand_qkv(99, 1, L, Hq, Hkv, D)
        q *= 1.5
        k *= 1.5
        want = pins.brute_force(q, k, v, w0, w_pre, 1e4, 1 / math.sqrt(D))
        got, _ = jo.bifocal_attention(q, k, v, w0, w_pre, 1e4, 1 / math.sqrt(D), block=5)
        if not np.allclose(got, want, atol=1e-12, rtol=0):
            return True
    return False


def test_unmutated_oracle_passes():
    assert not _pins_fail()


MUTANTS = {}


def mutant(fn):
    MUTANTS[fn.__name__] = fn
    return fn


@mutant
def rotation_sign_flipped(mp):
    orig = jo.rope_rotate
    mp.setattr(jo, "rope_rotate", lambda x, a, base: orig(x, -np.asarray(a), base))


@mutant
def group_size_floor(mp):
    mp.setattr(jo, "group_size", lambda L, w: max(1, L // w))


@mutant
def one_based_positions(mp):
    mp.setattr(jo, "correction_offset", lambda p, G: (np.asarray(p) + 1) // G - (np.asarray(p) + 1))


@mutant
def interleaved_pairs(mp):
    def rot(x, angle_pos, base):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[-1]
        ang = np.asarray(angle_pos, dtype=np.float64)[..., None] * jo.inv_freq(D, base)
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = a * s + b * c
        return out
    mp.setattr(jo, "rope_rotate", rot)


@mutant
def strict_window_edge(mp):
    orig = jo.bifocal_attention
    mp.setattr(jo, "bifocal_attention",
               lambda q, k, v, w0, *a, **kw: orig(q, k, v, w0 - 1, *a, **kw))


@mutant
def only_keys_aliased(mp):
    orig = jo.remote_view
    calls = {"n": 0}

    def rv(u, positions, G, base):
        calls["n"] += 1
        return orig(u, positions, G, base) if calls["n"] % 2 == 1 else np.asarray(u, np.float64)
    mp.setattr(jo, "remote_view", rv)


@mutant
def wrong_frequency_exponent(mp):
    mp.setattr(jo, "inv_freq", lambda D, base: np.float64(base) ** (-np.arange(D // 2) / D))


@mutant
def softmax_missing_max_shift_and_scale(mp):
    def sm(S, V):
        E = np.exp(S * 0.9)
        l = E.sum(axis=1, keepdims=True)
        return (E @ V) / l, np.log(l[:, 0])
    mp.setattr(jo, "softmax_rows", sm)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert _pins_fail(), f"planted mistake '{name}' went unnoticed"
