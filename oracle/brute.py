"""Pure-Python loop versions of the decode path for tiny shapes. Test infrastructure only.

Written independently of the vectorised oracle (no numpy in the arithmetic) so
that an indexing or transposition slip in one is caught by the other.
"""
from __future__ import annotations

import math


def rope_vec(x: list, pos: int, base: float) -> list:
    """Rotate-half RoPE of one vector: pairs (i, i + d/2) rotated by pos * base^(-2i/d)."""
    d = len(x)
    h = d // 2
    out = list(x)
    if base == 0:
        return out
    for i in range(h):
        ang = pos * base ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        out[i] = x[i] * c - x[i + h] * s
        out[i + h] = x[i + h] * c + x[i] * s
    return out


def attention(q: list, K: list, V: list, scale: float) -> list:
    scores = [scale * sum(qi * ki for qi, ki in zip(q, k)) for k in K]
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    return [sum(w[t] * V[t][e] for t in range(len(V))) / tot for e in range(len(V[0]))]


def palu_decode_one(hk: list, hv: list, Bk: list, q: list, col0: int, d_h: int,
                    theta: float, q_pos: int, scale: float) -> list:
    """One query head: K_t = hk_t B[:, col0:col0+d_h], RoPE at t, attention, p H^v."""
    T = len(hk)
    r = len(Bk)
    K = []
    for t in range(T):
        k = [sum(hk[t][i] * Bk[i][col0 + c] for i in range(r)) for c in range(d_h)]
        K.append(rope_vec(k, t, theta))
    qr = rope_vec(q, q_pos, theta)
    return attention(qr, K, hv, scale)
