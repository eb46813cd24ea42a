"""Seeded synthetic inputs for the bifocal attention workloads.

This module is shared by the float64 oracle's tests, the GPU parity tests,
``bench.py`` and the smoke entry.  It only draws random numbers and rounds
them to the storage dtype; it holds none of the attention method's
arithmetic (no RoPE, no schedule, no softmax).

Recipe (one NumPy ``Generator(PCG64(seed))`` per tensor set):
  * draw float32 N(0, 1) in the order q, k, v;
  * if the workload asks for a per-channel scale, draw one vector
    s ~ U(0.5, 2) of length D for each of q, k, v (in that order) and
    multiply it into the last axis;
  * if the workload asks for a global scale (1/sqrt(D)), multiply it in;
  * round to the storage dtype (bf16 with round-to-nearest-even, or keep
    float32).

The q and k drawn here stand for vectors that already carry ordinary RoPE
at their true positions (the KV cache "as stored"): a rotation of an
isotropic Gaussian has the same distribution, so no rotation is applied.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "DecodeWorkload", "DECODE_WORKLOAD",
    "bf16_bits_from_f32", "f32_from_bf16_bits", "make_prefill_inputs",
    "make_decode_prompt", "make_decode_step", "sampled_rows",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    dtype: str          # "f32" or "bf16"
    B: int
    L: int
    Hq: int
    Hkv: int
    D: int
    w0: int
    w_pretrained: int
    rope_base: float
    seed: int
    channel_scale: bool = False   # per-channel U(0.5, 2) scale per tensor
    global_scale: float = 1.0     # multiplied into q, k and v

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The workloads: a tiny fp32 case, the identity regime at L = w_pre,
# extension prefills at 64K (G = 2), 128K (G = 4) and 1M (G = 4), and a
# 128K decode.
WORKLOADS = {
    "tiny": Workload("tiny", "f32", 1, 512, 4, 2, 64, 64, 256, 1.0e4, 1001),
    "identity32k": Workload("identity32k", "bf16", 1, 32768, 16, 8, 128, 4096,
                            32768, 1.0e6, 1002, global_scale=1.0 / math.sqrt(128.0)),
    "ext64k": Workload("ext64k", "bf16", 1, 65536, 32, 8, 128, 4096, 32768,
                       1.0e6, 1003, channel_scale=True),
    "ext128k": Workload("ext128k", "bf16", 1, 131072, 32, 8, 128, 4096, 32768,
                        1.0e6, 1004),
    # a 256K-native model extended 4x to 1M tokens (G = 4), one KV head and
    # its 4 query heads: one GPU's share of an 8-KV-head model split by head
    "ext1m": Workload("ext1m", "bf16", 1, 1048576, 4, 1, 128, 4096, 262144,
                      1.0e6, 1006),
}


@dataclasses.dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    prompt_len: int     # keys already in the cache before the first step
    steps: int          # decode steps; step s appends position prompt_len-1+s
    Hq: int
    Hkv: int
    D: int
    w0: int
    w_pretrained: int
    rope_base: float
    seed: int

    @property
    def Lmax(self) -> int:
        return self.prompt_len + self.steps

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


DECODE_WORKLOAD = DecodeWorkload("decode128k", 1, 131072, 256, 32, 8, 128, 4096,
                                 32768, 1.0e6, 1005)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _finish(x32: np.ndarray, dtype: str):
    """Return (storage array, exact float64 value of the storage)."""
    if dtype == "bf16":
        bits = bf16_bits_from_f32(x32)
        return bits, f32_from_bf16_bits(bits).astype(np.float64)
    if dtype == "f32":
        x32 = np.ascontiguousarray(x32, dtype=np.float32)
        return x32, x32.astype(np.float64)
    raise ValueError(dtype)


def make_prefill_inputs(w: Workload, L: int | None = None, want_f64: bool = True):
    """Seeded q [B,L,Hq,D], k and v [B,L,Hkv,D].

    Returns a dict with storage arrays ``q, k, v`` (uint16 bf16 bits or
    float32) and, if ``want_f64``, their exact float64 values ``q64, k64, v64``.
    ``L`` overrides the workload length (the draw order stays the same, so a
    shorter L is not a prefix of the longer one).
    """
    L = w.L if L is None else L
    rng = np.random.Generator(np.random.PCG64(w.seed))
    q = rng.standard_normal((w.B, L, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, L, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, L, w.Hkv, w.D), dtype=np.float32)
    if w.channel_scale:
        for x in (q, k, v):
            s = rng.uniform(0.5, 2.0, size=w.D).astype(np.float32)
            x *= s
    if w.global_scale != 1.0:
        g = np.float32(w.global_scale)
        q *= g
        k *= g
        v *= g
    out = {}
    for name, x in (("q", q), ("k", k), ("v", v)):
        st, x64 = _finish(x, w.dtype)
        out[name] = st
        if want_f64:
            out[name + "64"] = x64
    return out


def make_decode_prompt(w: DecodeWorkload):
    """bf16 caches [B, Lmax, Hkv, D]; rows < prompt_len seeded, the rest zero."""
    rng = np.random.Generator(np.random.PCG64(w.seed))
    kc = np.zeros((w.B, w.Lmax, w.Hkv, w.D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    shape = (w.B, w.prompt_len, w.Hkv, w.D)
    kc[:, :w.prompt_len] = bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    vc[:, :w.prompt_len] = bf16_bits_from_f32(rng.standard_normal(shape, dtype=np.float32))
    return kc, vc


def make_decode_step(w: DecodeWorkload, s: int):
    """Step s (1-based): new query [B,1,Hq,D] and new k/v rows [B,1,Hkv,D], bf16 bits.

    The caller writes the new k/v row at position prompt_len - 1 + s and the
    step attends the L = prompt_len + s keys at positions 0 .. L-1.
    """
    rng = np.random.Generator(np.random.PCG64([w.seed, s]))
    q = bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hq, w.D), dtype=np.float32))
    k = bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hkv, w.D), dtype=np.float32))
    v = bf16_bits_from_f32(rng.standard_normal((w.B, 1, w.Hkv, w.D), dtype=np.float32))
    return q, k, v


def sampled_rows(L: int, w0: int, w_pretrained: int, n_random: int, seed: int,
                 tile: int = 64) -> np.ndarray:
    """Structural query rows plus seeded uniform rows, sorted and unique.

    Structural rows: the first rows, the rows around the local-window edge
    w0, around every multiple of the pretrained window below L, the last
    rows, and the first/last row of the tiles next to each of those.
    """
    pts = {0, 1, 2, L - 2, L - 1}
    edges = [m + d for m in range(w_pretrained, L, w_pretrained) for d in (-1, 0)]
    for c in [w0 - 1, w0, w0 + 1, w0 + 2] + edges:
        pts.add(c)
        t = (c // tile) * tile
        pts.update({t - 1, t, t + tile - 1, t + tile})
    rng = np.random.Generator(np.random.PCG64([seed, 7]))
    if n_random:
        pts.update(rng.integers(0, L, size=n_random).tolist())
    return np.array(sorted(p for p in pts if 0 <= p < L), dtype=np.int64)
