"""Test-side helpers for the GPU parity tests: reading the library's documented
cache layouts back into plain [B][U][T][r] arrays, and the error metric.

These are index permutations and nibble extraction only (the layouts are
specified in include/lrkv.h); they hold no step of the decode path."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(msg: str) -> None:
    """Print and flush what names the case before a GPU step."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def rel_l2(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||got - ref|| / ||ref|| over the last axis, per leading index."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return np.linalg.norm(got - ref, axis=-1) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def hv_fp16_tokens(hv: torch.Tensor) -> np.ndarray:
    """[B][U][cap/32][r][32] half -> [B][U][cap][r] float16."""
    a = hv.cpu().numpy()
    B, U, nb, r, _ = a.shape
    return a.transpose(0, 1, 2, 4, 3).reshape(B, U, nb * 32, r)


def _nibbles(byte_arr: np.ndarray) -> np.ndarray:
    b = byte_arr.astype(np.int16)
    lo = b & 0xF
    hi = (b >> 4) & 0xF
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def hk_int4_codes(hk: torch.Tensor) -> np.ndarray:
    """[B][U][cap][r/2] uint8 -> codes [B][U][cap][r] (dim 2i low nibble)."""
    return _nibbles(hk.cpu().numpy())


def hv_int4_codes(hv: torch.Tensor) -> np.ndarray:
    """[B][U][cap/32][r][16] uint8 -> codes [B][U][cap][r] (token 2i low nibble)."""
    c = _nibbles(hv.cpu().numpy())                 # [B][U][nb][r][32]
    B, U, nb, r, _ = c.shape
    return c.transpose(0, 1, 2, 4, 3).reshape(B, U, nb * 32, r)


def sv_tokens(sv: torch.Tensor) -> np.ndarray:
    """[B][U][cap/32][r/32][32] half -> [B][U][cap][r/32]."""
    a = sv.cpu().numpy()
    B, U, nb, g, _ = a.shape
    return a.transpose(0, 1, 2, 4, 3).reshape(B, U, nb * 32, g)
