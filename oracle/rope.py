"""Rotary position embedding, rotate-half convention, float64. Test infrastructure only.

The Palu digest (Method details) says RoPE is applied to queries and keys before
their product but prints no formula. The Shard post (section 5, "undo RoPE")
prints the rotate-half form used by Llama: rotate_half([a, b]) = [-b, a] within
each head's slice, with cos/sin of (position * theta_i). The frequencies
theta_i = base^(-2 i / d_h), i < d_h / 2, repeated over both halves, are the
RoFormer/Llama schedule (a reading: the pages name the base, not the schedule).
"""
from __future__ import annotations

import numpy as np


def freqs(d_h: int, base: float) -> np.ndarray:
    """theta_i = base^(-2 i / d_h) for i < d_h/2 (float64)."""
    i = np.arange(d_h // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d_h)


def _angles(pos, d_h: int, base: float) -> np.ndarray:
    pos = np.asarray(pos, dtype=np.float64)
    return pos[..., None] * freqs(d_h, base)           # [..., d_h/2]


def rotate_half(x: np.ndarray) -> np.ndarray:
    h = x.shape[-1] // 2
    return np.concatenate([-x[..., h:], x[..., :h]], axis=-1)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """x' = x * cos + rotate_half(x) * sin at integer positions ``pos`` (broadcast over
    the leading axes of x). base == 0 means no rotation."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    ang = _angles(pos, x.shape[-1], base)
    c = np.cos(np.concatenate([ang, ang], axis=-1))
    s = np.sin(np.concatenate([ang, ang], axis=-1))
    return x * c + rotate_half(x) * s


def unrope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Inverse rotation x = x' * cos - rotate_half(x') * sin (Shard, section 5, step 1)."""
    x = np.asarray(x, dtype=np.float64)
    if base == 0:
        return x.copy()
    ang = _angles(pos, x.shape[-1], base)
    c = np.cos(np.concatenate([ang, ang], axis=-1))
    s = np.sin(np.concatenate([ang, ang], axis=-1))
    return x * c - rotate_half(x) * s
