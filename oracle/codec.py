"""Symmetric int4 latent codec, one fp16 scale per 32 consecutive elements of a token.

Test infrastructure only. This is the one oracle module that is not float64: the
quantiser is defined by fixed fp32 / fp16 steps, and the oracle performs exactly
those steps with numpy float32 / float16 scalars so that codes and scales can be
compared bit for bit.

Sources: the Palu digest (Supplementary details, KV-cache compression) uses plain per-token
quantisation and cites group-of-32 fine-grained grouping; the Shard post
(section 5, step 4) quantises coefficients to symmetric int4 in [-7, 7] with a
scale per component. Reading used here (the pages fix no rounding rule):

  amax  = max |x| over the 32-element group            (fp32, exact)
  s32   = amax / 7                                     (fp32 IEEE division, RNE)
  s16   = fp16(s32), round-to-nearest-even; +inf saturates to 65504
  code  = clamp(round_half_even(x / s16), -7, 7), the quotient formed in fp64
          (exact enough that ties k + 1/2 are decided exactly); s16 == 0 -> 0
  pack  = element 2i in the low nibble, 2i+1 in the high nibble, 4-bit two's
          complement
  x_hat = code * s16 evaluated in fp32 (exact)
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def quantize(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """x float32 [..., r] (r % 32 == 0) -> (codes int8 [..., r], scales float16 [..., r/32])."""
    x = np.asarray(x, dtype=np.float32)
    r = x.shape[-1]
    if r % GROUP:
        raise ValueError("last dimension must be a multiple of 32")
    g = x.reshape(x.shape[:-1] + (r // GROUP, GROUP))
    amax = np.max(np.abs(g), axis=-1)                       # float32
    s32 = (amax / np.float32(7.0)).astype(np.float32)       # IEEE fp32 division
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)                        # RNE
    s16 = np.where(np.isinf(s16), np.float16(65504.0), s16).astype(np.float16)
    den = s16.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = g.astype(np.float64) / den
    codes = np.clip(np.rint(q), -7, 7)                      # rint: half to even
    codes = np.where(den == 0.0, 0.0, codes)
    return codes.astype(np.int8).reshape(x.shape), s16


def pack(codes: np.ndarray) -> np.ndarray:
    """int8 codes [..., r] -> uint8 [..., r/2]; element 2i low nibble, 2i+1 high nibble."""
    c = np.asarray(codes).astype(np.int16) & 0xF
    lo = c[..., 0::2]
    hi = c[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    """uint8 [..., r/2] -> int8 codes [..., r] (sign-extended nibbles)."""
    p = np.asarray(packed).astype(np.int16)
    lo = p & 0xF
    hi = (p >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """code * s16 in fp32 (exact): codes [..., r], scales [..., r/32] -> float32 [..., r]."""
    c = np.asarray(codes).astype(np.float32)
    s = np.repeat(np.asarray(scales).astype(np.float32), GROUP, axis=-1)
    return (c * s).astype(np.float32)
