"""Plain float64 definition of Jet-Long bifocal RoPE attention (oracle).

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU
baseline leg of the benchmark, never by the product path.

Source: "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
RoPE" (Tang, Wang, Gu, Han, Cai), §3 and its equations:

  * §3, score rule (Eq. 1): a query at position q and a key at position k
    score with their ordinary RoPE vectors when q - k <= w0, and with both
    positions passed through the aliasing map f when q - k > w0.
  * §3.1, group size (Eq. 2): G = max(1, ceil(L / w_pretrained)).
  * §3.1, aliasing map (Eq. 3): f(x) = floor(x / G).
  * §3.2, cache (Eq. 4): the cache holds RoPE(x_k, k), never rewritten.
  * §3.2, correction (Eq. 5): dq = f(q) - q, dk = f(k) - k; rotating a stored
    RoPE vector by its offset gives the remote view.
  * §3.3, inclusion-exclusion merge (Eq. 6): the output is assembled from
    three normalised attention partials A, B, C with weights W_X.

Readings where the pages leave a step open (each listed in the design notes):
positions are 0-based; L is the number of tokens in the call, one G per
call; the window edge is inclusive (local iff q - k <= w0); attention is
causal (k <= q); both q and k are aliased; RoPE pairs channel i with
channel i + D/2 and uses theta_i = base^(-2i/D); the softmax scale is an
explicit argument with no extra temperature; query head h reads KV head
h // (Hq / Hkv).  For the merge, A = local view over the local keys, B =
remote view over all causal keys, C = remote view over the local keys.

Everything is float64.  Score blocks are formed explicitly as dense
[rows x keys] matrices; matmul is the only library primitive used.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "group_size", "alias_position", "correction_offset", "inv_freq",
    "rope_rotate", "remote_view", "softmax_rows", "bifocal_attention",
    "plain_causal_attention", "decode_attention", "inclusion_exclusion_attention",
    "fi_scale", "fi_ramp", "fi_inv_freq", "fi_remote_view", "bifocal_attention_fi",
    "decode_attention_fi",
]


# ---------------------------------------------------------------- schedule
def group_size(L: int, w_pretrained: int) -> int:
    """§3.1 Eq. (2): G = max(1, ceil(L / w_pretrained)), integer arithmetic."""
    L = int(L)
    w_pretrained = int(w_pretrained)
    if L < 1 or w_pretrained < 1:
        raise ValueError("L and w_pretrained must be >= 1")
    return max(1, -(-L // w_pretrained))


def alias_position(p, G: int):
    """§3.1 Eq. (3): f(x) = floor(x / G) for non-negative integer positions."""
    return np.asarray(p, dtype=np.int64) // int(G)


def correction_offset(p, G: int):
    """§3.2 Eq. (5): the offset f(p) - p that moves a stored RoPE phase to f(p)."""
    p = np.asarray(p, dtype=np.int64)
    return alias_position(p, G) - p


# -------------------------------------------------------------------- RoPE
def inv_freq(D: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i = 0 .. D/2-1 (rotate-half RoPE frequencies)."""
    i = np.arange(D // 2, dtype=np.float64)
    return np.float64(base) ** (-(2.0 * i) / np.float64(D))


def rope_rotate(x: np.ndarray, angle_pos, base: float) -> np.ndarray:
    """Rotate each channel pair (i, i + D/2) of x by angle_pos * theta_i.

    ``angle_pos`` broadcasts against ``x.shape[:-1]`` (integer positions or
    position offsets).  (a, b) -> (a cos - b sin, a sin + b cos).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    ang = np.asarray(angle_pos, dtype=np.float64)[..., None] * inv_freq(D, base)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def remote_view(u: np.ndarray, positions, G: int, base: float) -> np.ndarray:
    """§3.2: rotate stored vectors u[B, n, H, D] at ``positions`` [n] by their
    correction offsets, giving RoPE(x, f(p)) from the stored RoPE(x, p)."""
    off = correction_offset(positions, G)
    return rope_rotate(u, off[None, :, None], base)


# ----------------------------------------------------------------- softmax
def softmax_rows(S: np.ndarray, V: np.ndarray):
    """Row softmax of a dense score block S [R, K] (masked entries = -inf)
    applied to V [K, D].  Returns (out [R, D], natural-log LSE [R])."""
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    out = (E @ V) / l
    return out, m[:, 0] + np.log(l[:, 0])


# ---------------------------------------------------------- core (dense)
def _attend(qv, q_pos, k, v, G, w0, base, sm_scale, bifocal, block, remote=None):
    """Dense bifocal (or plain) causal attention for the query vectors
    qv [B, n, Hq, D] at positions q_pos [n] over keys 0..Lk-1.  ``remote``
    (u, positions) -> remote view; by default the aliased view under G."""
    B, n, Hq, D = qv.shape
    Lk, Hkv = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    R = Hq // Hkv
    q_pos = np.asarray(q_pos, dtype=np.int64)
    if remote is None:
        remote = lambda u, pos: remote_view(u, pos, G, base)
    if bifocal:
        k_rem = remote(k, np.arange(Lk))
        q_rem = remote(qv, q_pos)
    out = np.empty((B, n, Hq, D), dtype=np.float64)
    lse = np.empty((B, Hq, n), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // R
            for s in range(0, n, block):
                rp = q_pos[s:s + block]
                kend = int(rp.max()) + 1           # keys beyond every row are masked
                dist = rp[:, None] - np.arange(kend)[None, :]
                S = (qv[b, s:s + block, h] @ k[b, :kend, g].T) * sm_scale
                if bifocal:
                    S_rem = (q_rem[b, s:s + block, h] @ k_rem[b, :kend, g].T) * sm_scale
                    S = np.where(dist <= w0, S, S_rem)
                S[dist < 0] = -np.inf
                o, ls = softmax_rows(S, v[b, :kend, g])
                out[b, s:s + block, h] = o
                lse[b, h, s:s + block] = ls
    return out, lse


def bifocal_attention(q, k, v, w0: int, w_pretrained: int, rope_base: float,
                      sm_scale: float, rows=None, block: int = 64):
    """Prefill: q [B,L,Hq,D], k/v [B,L,Hkv,D] (stored RoPE vectors), causal.

    Returns (out [B, n, Hq, D], lse [B, Hq, n]) for the query ``rows``
    (default: all L).  G is fixed by the full length L of the call.
    """
    q = np.asarray(q, dtype=np.float64)
    L = q.shape[1]
    G = group_size(L, w_pretrained)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    return _attend(q[:, rows], rows, np.asarray(k, np.float64), np.asarray(v, np.float64),
                   G, int(w0), rope_base, sm_scale, True, block)


def plain_causal_attention(q, k, v, sm_scale: float, rows=None, block: int = 64):
    """Ordinary causal attention on the stored RoPE vectors (the base model)."""
    q = np.asarray(q, dtype=np.float64)
    L = q.shape[1]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    return _attend(q[:, rows], rows, np.asarray(k, np.float64), np.asarray(v, np.float64),
                   1, 0, 0.0, sm_scale, False, block)


def decode_attention(q_tok, k_cache, v_cache, L: int, w0: int, w_pretrained: int,
                     rope_base: float, sm_scale: float):
    """One decode step: query q_tok [B,Hq,D] at position L-1 against cache
    rows 0..L-1 (the new token's k/v already written at row L-1).  G is
    recomputed from L (§3.2: cached keys are reinterpreted under the current
    G).  Returns (out [B,Hq,D], lse [B,Hq])."""
    q_tok = np.asarray(q_tok, dtype=np.float64)
    G = group_size(L, w_pretrained)
    o, ls = _attend(q_tok[:, None], np.array([L - 1]),
                    np.asarray(k_cache[:, :L], np.float64),
                    np.asarray(v_cache[:, :L], np.float64),
                    G, int(w0), rope_base, sm_scale, True, 1)
    return o[:, 0], ls[:, :, 0]


# ------------------------------------------------- §3.3 three-pass merge
def inclusion_exclusion_attention(q, k, v, w0: int, w_pretrained: int,
                                  rope_base: float, sm_scale: float, rows=None):
    """§3.3 Eq. (6) taken literally: three separately normalised attention
    passes, A (local view, local keys), B (remote view, all causal keys),
    C (remote view, local keys), merged as
        O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C),
    with W_X the softmax denominator of pass X.  The weights are carried as
    log-sum-exps and shifted by their maximum before exponentiation."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, L, Hq, D = q.shape
    Hkv = k.shape[2]
    R = Hq // Hkv
    G = group_size(L, w_pretrained)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    k_rem = remote_view(k, np.arange(L), G, rope_base)
    q_rem = remote_view(q[:, rows], rows, G, rope_base)
    out = np.empty((B, len(rows), Hq, D))
    for b in range(B):
        for h in range(Hq):
            g = h // R
            dist = rows[:, None] - np.arange(L)[None, :]
            causal = dist >= 0
            local = causal & (dist <= w0)
            S_loc = (q[b, rows, h] @ k[b, :, g].T) * sm_scale
            S_rem = (q_rem[b, :, h] @ k_rem[b, :, g].T) * sm_scale
            parts = []
            for S, mask in ((S_loc, local), (S_rem, causal), (S_rem, local)):
                Sm = np.where(mask, S, -np.inf)
                o, ls = softmax_rows(Sm, v[b, :, g])
                parts.append((o, ls))
            (oA, lA), (oB, lB), (oC, lC) = parts
            M = np.maximum(np.maximum(lA, lB), lC)
            wA, wB, wC = np.exp(lA - M), np.exp(lB - M), np.exp(lC - M)
            num = wA[:, None] * oA + wB[:, None] * oB - wC[:, None] * oC
            out[b, :, h] = num / (wA + wB - wC)[:, None]
    return out


# ------------------------- §4.7 ablation: frequency interpolation (remote)
# The remote view moves each stored phase p*theta_i to p*theta'_i, where
# theta' are YaRN-style interpolated frequencies for the continuous ratio
# s = max(1, L / w_pretrained) of §3.1.  The local window is unchanged.  The
# pages do not give the ramp; the reading here is YaRN's: with
# r_i = w_pretrained / lambda_i (turns of pair i over the pretrained window,
# lambda_i = 2 pi / theta_i), gamma_i = 0 for r_i < alpha (interpolated:
# theta_i / s), 1 for r_i > beta (kept: theta_i), linear in between; no
# attention temperature.
def fi_scale(L: int, w_pretrained: int) -> float:
    """§3.1: the continuous scaling ratio s = max(1, L / w_pretrained)."""
    return max(1.0, float(L) / float(w_pretrained))


def fi_ramp(D: int, base: float, w_pretrained: int, alpha: float, beta: float) -> np.ndarray:
    """gamma_i in [0, 1] for each rotation pair (see the note above)."""
    r = float(w_pretrained) * inv_freq(D, base) / (2.0 * np.pi)
    return np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)


def fi_inv_freq(D: int, base: float, L: int, w_pretrained: int, alpha: float, beta: float) -> np.ndarray:
    """theta'_i = (1 - gamma_i) theta_i / s + gamma_i theta_i."""
    theta = inv_freq(D, base)
    g = fi_ramp(D, base, w_pretrained, alpha, beta)
    return (1.0 - g) * theta / fi_scale(L, w_pretrained) + g * theta


def fi_remote_view(u: np.ndarray, positions, L: int, w_pretrained: int, base: float,
                   alpha: float, beta: float) -> np.ndarray:
    """Stored vectors u[B, n, H, D] = RoPE(x, p) at ``positions`` moved to the
    interpolated phase: pair i rotated by p (theta'_i - theta_i)."""
    u = np.asarray(u, dtype=np.float64)
    D = u.shape[-1]
    dtheta = fi_inv_freq(D, base, L, w_pretrained, alpha, beta) - inv_freq(D, base)
    ang = np.asarray(positions, dtype=np.float64)[None, :, None, None] * dtheta
    c, s = np.cos(ang), np.sin(ang)
    a, b = u[..., : D // 2], u[..., D // 2:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=-1)


def bifocal_attention_fi(q, k, v, w0: int, w_pretrained: int, rope_base: float, alpha: float,
                         beta: float, sm_scale: float, rows=None, block: int = 64):
    """Prefill with the interpolated remote view: the score rule of §3 Eq. 1
    (stored vectors when q - k <= w0) with the remote pairs scored in the
    frequency-interpolation view for this call's L.  Returns (out, lse) as
    bifocal_attention."""
    q = np.asarray(q, dtype=np.float64)
    L = q.shape[1]
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    remote = lambda u, pos: fi_remote_view(u, pos, L, w_pretrained, rope_base, alpha, beta)
    return _attend(q[:, rows], rows, np.asarray(k, np.float64), np.asarray(v, np.float64),
                   0, int(w0), rope_base, sm_scale, True, block, remote)


def decode_attention_fi(q_tok, k_cache, v_cache, L: int, w0: int, w_pretrained: int,
                        rope_base: float, alpha: float, beta: float, sm_scale: float):
    """One decode step with the interpolated remote view, s from this L."""
    q_tok = np.asarray(q_tok, dtype=np.float64)
    remote = lambda u, pos: fi_remote_view(u, pos, L, w_pretrained, rope_base, alpha, beta)
    o, ls = _attend(q_tok[:, None], np.array([L - 1]),
                    np.asarray(k_cache[:, :L], np.float64),
                    np.asarray(v_cache[:, :L], np.float64),
                    0, int(w0), rope_base, sm_scale, True, 1, remote)
    return o[:, 0], ls[:, :, 0]
