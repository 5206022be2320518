"""Seeded synthetic inputs shaped like the workloads of the low-rank KV pages.

This module is shared by the tests, the oracle checks and ``bench.py``. It holds
random draws and their scaling only: no step of the decode path (no fp16/int4
conversion of latents, no reconstruction, no RoPE, no softmax, no page
factorisation) lives here. Every generator takes an explicit seed and uses
numpy's PCG64 ``default_rng``.

Workload recipes (shapes from the pages, distributions stated where the pages
are silent):

* ``palu_tiny``      -- tiny G-LRD layer: d_model 256, 4 heads of 64, groups of
                        two heads, per-group K/V weight ``U diag(s) V^T`` with
                        Haar-orthogonal U, V and ``s_i = exp(-i/24)``.
* ``latent_layer``   -- latents and reconstruction matrices of a layer whose
                        per-group weight has singular values ``exp(-i/tau)``.
                        Latents are drawn as ``sqrt(s_i) * z`` which is exactly
                        the distribution of ``x A`` for ``x ~ N(0, I)`` and
                        ``A = U_r sqrt(S_r)`` with orthonormal ``U_r``.
* ``hadamard_mixed`` -- the same latents/basis expressed in a 2^k-point
                        Sylvester-Hadamard mixed basis (the int4 workload stores
                        latents in that basis).
* ``paged_dense``    -- dense per-head K/V with rank-12 structure plus noise.
* ``factored_pages`` -- random page factors (orthonormal L, scaled R).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "haar_orthonormal", "palu_tiny", "latent_layer", "hadamard_mixed",
    "queries", "paged_dense", "factored_pages", "sylvester",
]


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def haar_orthonormal(rng: np.random.Generator, n: int, k: int | None = None) -> np.ndarray:
    """n x k matrix with Haar-distributed orthonormal columns (QR of a Gaussian, sign-fixed)."""
    k = n if k is None else k
    g = rng.standard_normal((n, k))
    q, r = np.linalg.qr(g)
    q *= np.sign(np.diag(r))[None, :]
    return q


def sylvester(n: int) -> np.ndarray:
    """Unnormalised Sylvester-order Hadamard matrix of size n (a power of two)."""
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    if h.shape[0] != n:
        raise ValueError("n must be a power of two")
    return h


def palu_tiny(seed: int = 1, T: int = 256, full_rank_factors: bool = True) -> dict:
    """Tiny G-LRD attention layer (d_model 256, 4 heads, d_h 64, groups of 2).

    Returns the raw weights of the layer (the oracle factors them itself) plus
    the true factors used to build them, the input tokens ``x`` and the query
    and output projections.
    """
    rng = _rng(seed)
    d_model, n_heads, d_h, s = 256, 4, 64, 2
    groups = n_heads // s
    width = s * d_h
    sv = np.exp(-np.arange(width) / 24.0)
    out = {"d_model": d_model, "n_heads": n_heads, "d_h": d_h, "s": s, "sv": sv}
    for kind in ("k", "v"):
        Us, Vs, Ws = [], [], []
        for _ in range(groups):
            U = haar_orthonormal(rng, d_model, width)
            V = haar_orthonormal(rng, width, width)
            Us.append(U)
            Vs.append(V)
            Ws.append((U * sv[None, :]) @ V.T)
        out["U_" + kind] = np.stack(Us)
        out["V_" + kind] = np.stack(Vs)
        out["W_" + kind] = np.stack(Ws)          # [groups][d_model][s*d_h]
    out["W_q"] = rng.standard_normal((d_model, d_model)) / np.sqrt(d_model)
    out["W_o"] = rng.standard_normal((d_model, d_model)) / np.sqrt(d_model)
    out["x"] = rng.standard_normal((T, d_model))
    return out


def latent_layer(seed: int, batch: int, units: int, T: int, rank: int, width: int,
                 tau: float, dtype=np.float32) -> dict:
    """Latent caches and reconstruction matrices of one low-rank attention layer.

    ``units`` groups (or KV heads), each with ``width`` = s*d_h output columns
    and rank ``rank``. Singular values ``s_i = exp(-i/tau)`` for i < width.
    Returns ``hk, hv`` [batch][units][T][rank] (``dtype``), ``Bk, Bv``
    [units][rank][width] as float16 (the stored weight precision) and ``sv``.
    """
    rng = _rng(seed)
    sv = np.exp(-np.arange(width) / float(tau))
    root = np.sqrt(sv[:rank])
    Bs = {}
    for kind in ("k", "v"):
        mats = []
        for _ in range(units):
            V = haar_orthonormal(rng, width, rank)          # width x rank
            mats.append((root[:, None] * V.T).astype(np.float16))
        Bs[kind] = np.ascontiguousarray(np.stack(mats))     # C order (V.T would leave it strided)
    hk = rng.standard_normal((batch, units, T, rank), dtype=np.float32)
    hk *= root.astype(np.float32)
    hv = rng.standard_normal((batch, units, T, rank), dtype=np.float32)
    hv *= root.astype(np.float32)
    return {"hk": hk.astype(dtype, copy=False), "hv": hv.astype(dtype, copy=False),
            "Bk": Bs["k"], "Bv": Bs["v"], "sv": sv}


def hadamard_mixed(h: np.ndarray, B: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Express latents ``h`` [..., r] and basis ``B`` [units][r][w] in the Sylvester-
    Hadamard mixed basis (entries +-1/sqrt(r)). ``h @ B`` is unchanged up to
    rounding. Used to synthesise the int4 workload whose latents are stored in
    that basis."""
    r = h.shape[-1]
    H = sylvester(r) / np.sqrt(r)
    hm = (h.astype(np.float64) @ H).astype(np.float32)
    Bm = np.einsum("ij,ujw->uiw", H, B.astype(np.float64)).astype(np.float16)
    return hm, np.ascontiguousarray(Bm)


def queries(seed: int, batch: int, heads: int, dim: int, scale: float = 1.0) -> np.ndarray:
    """Query vectors ~ N(0, scale^2), float32 [batch][heads][dim]."""
    rng = _rng(seed)
    return (rng.standard_normal((batch, heads, dim)) * scale).astype(np.float32)


def paged_dense(seed: int, batch: int, kv_heads: int, T: int, d: int = 128,
                signal_rank: int = 12, noise_std: float = 0.05) -> dict:
    """Dense per-head K/V = Z C + noise_std * N with Z ~ N(0,1)^{T x k} and
    C ~ N(0, 1/k)^{k x d} (unit signal variance). float16 [batch][kv_heads][T][d]."""
    rng = _rng(seed)
    out = {}
    for kind in ("k", "v"):
        arr = np.empty((batch, kv_heads, T, d), dtype=np.float16)
        for b in range(batch):
            for h in range(kv_heads):
                Z = rng.standard_normal((T, signal_rank), dtype=np.float32)
                C = rng.standard_normal((signal_rank, d), dtype=np.float32) / np.float32(np.sqrt(signal_rank))
                N = rng.standard_normal((T, d), dtype=np.float32)
                arr[b, h] = (Z @ C + np.float32(noise_std) * N).astype(np.float16)
        out[kind] = arr
    return out


def factored_pages(seed: int, n: int, P: int, d: int, r: int) -> dict:
    """Random factored pages: L [n][P][r] with orthonormal columns, R [n][r][d] with
    decreasing row norms, both float16. L R has roughly unit-variance entries."""
    rng = _rng(seed)
    L = np.empty((n, P, r), dtype=np.float16)
    R = np.empty((n, r, d), dtype=np.float16)
    sig = np.sqrt(P * d / r) * np.exp(-np.arange(r) / 8.0)
    sig *= np.sqrt(P * d / np.sum(sig ** 2))
    for i in range(n):
        L[i] = haar_orthonormal(rng, P, r).astype(np.float16)
        W = haar_orthonormal(rng, d, r)
        R[i] = (sig[:, None] * W.T).astype(np.float16)
    return {"L": L, "R": R}
