"""Byte accounting of dense and compressed KV caches. Test infrastructure only."""
from __future__ import annotations


def kv_bytes(layers: int, kv_heads: int, head_dim: int, T: int, bytes_per_elem: int) -> int:
    """2 L H_kv d T bytes: one request's dense K and V (PuzzleKV section 1; Shard section 1)."""
    return 2 * layers * kv_heads * head_dim * T * bytes_per_elem


def latent_bytes(batch: int, units: int, T: int, rank: int, fmt: str = "fp16") -> int:
    """Bytes one decode step must read from a latent cache (K and V latents of every token).

    fp16: r halves per token and side. int4 (groups of 32): r/2 code bytes plus one
    fp16 scale per 32 elements."""
    if fmt == "fp16":
        per_side = rank * 2
    elif fmt == "int4":
        per_side = rank // 2 + 2 * (rank // 32)
    else:
        raise ValueError(fmt)
    return 2 * batch * units * T * per_side


def paged_bytes(batch: int, kv_heads: int, dense_pages: int, factored_pages: int,
                P: int, d: int, r_k: int, r_v: int, elem: int = 2) -> int:
    """Bytes one hybrid decode step reads: dense pages (K and V, P x d each) plus the
    factors of factored pages (L: P x r, R: r x d for each of K and V)."""
    dense = dense_pages * 2 * P * d * elem
    fact = factored_pages * ((P + d) * r_k + (P + d) * r_v) * elem
    return batch * kv_heads * (dense + fact)
