"""Offline weight preparation (float64). Test infrastructure only.

Row-vector convention throughout: a latent is ``h = x A`` and a reconstruction
is ``y = h B`` (the Palu digest writes both ``h = A x`` and ``y = x A B``; the
row form is the one its fusion identities use).
"""
from __future__ import annotations

import numpy as np


def svd_factor(W: np.ndarray, r: int) -> tuple[np.ndarray, np.ndarray]:
    """Rank-r factors of W (m x n): A = U_r sqrt(S_r), B = sqrt(S_r) V_r^T.

    Palu digest, Background ("SVD for low-rank approximation"): W ~ A B with the
    square root of the r largest singular values split between the two factors.
    """
    U, S, Vt = np.linalg.svd(np.asarray(W, dtype=np.float64), full_matrices=False)
    root = np.sqrt(S[:r])
    return U[:, :r] * root[None, :], root[:, None] * Vt[:r, :]


def factor_storage_ratio(m: int, n: int, r: int) -> float:
    """(m r + r n) / (m n): storage of the two factors relative to W (Palu digest, Background)."""
    return (m * r + r * n) / (m * n)


def group_heads(W_heads: list[np.ndarray], s: int) -> list[np.ndarray]:
    """Concatenate consecutive per-head weights [d x d_h] into groups of s heads.

    Palu digest, Method details (G-LRD): W_g = [W_{j,1} ... W_{j,s}] in R^{d x s d_h}.
    """
    if len(W_heads) % s:
        raise ValueError("number of heads must be a multiple of the group size")
    return [np.concatenate(W_heads[g:g + s], axis=1) for g in range(0, len(W_heads), s)]


def glrd_factor(W_groups: list[np.ndarray], r: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-group truncated SVD (G-LRD): returns A [G][d][r] and B [G][r][s d_h]."""
    As, Bs = zip(*(svd_factor(W, r) for W in W_groups))
    return np.stack(As), np.stack(Bs)


def hadamard(n: int) -> np.ndarray:
    """Orthonormal Walsh-Hadamard matrix in Sylvester (natural) order, H / sqrt(n).

    Palu digest, Method details (Hadamard transform removes latent outliers). The
    pages do not fix size or order; Sylvester order without random signs is used.
    """
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    if H.shape[0] != n:
        raise ValueError("n must be a power of two")
    return H / np.sqrt(n)


def fwht(x: np.ndarray) -> np.ndarray:
    """Fast butterfly Walsh-Hadamard transform along the last axis, scaled by 1/sqrt(n).
    Equals ``x @ hadamard(n)`` (the matrix is symmetric)."""
    y = np.array(x, dtype=np.float64, copy=True)
    n = y.shape[-1]
    h = 1
    while h < n:
        y = y.reshape(y.shape[:-1] + (n // (2 * h), 2, h))
        a = y[..., 0, :].copy()
        b = y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (n,))
        h *= 2
    return y / np.sqrt(n)


def hadamard_fold(A: np.ndarray, B: np.ndarray, R: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """W ~ A B = (A R)(R^T B) (Palu digest, Method details: Hadamard folded into the factors)."""
    return A @ R, R.T @ B


def latent_project(x: np.ndarray, A_units: np.ndarray) -> np.ndarray:
    """Latents of every unit for tokens x [n][d]: h[t][u] = x_t A_u, A_units [U][d][r] -> [n][U][r].

    Palu digest, Method details: the cache stores h = x A in place of keys and values.
    """
    x = np.asarray(x, dtype=np.float64)
    A = np.asarray(A_units, dtype=np.float64)
    return np.stack([x @ A[u] for u in range(A.shape[0])], axis=1)


def fuse_v_into_wo(Bv_head: np.ndarray, Wo_head: np.ndarray) -> np.ndarray:
    """B^v_i W^o_i (r x d): value reconstruction absorbed into the output projection.

    Palu digest, Method details: a_i W^o_i = p_i H^v_i (B^v_i W^o_i).
    """
    return Bv_head @ Wo_head


def fuse_k_into_wq(Wq_head: np.ndarray, Bk_head: np.ndarray) -> np.ndarray:
    """W^q_i (B^k_i)^T (d x r): key reconstruction absorbed into the query projection.

    Palu digest, Method details: q_i K_i^T = x_t (W^q_i (B^k_i)^T) (H^k_i)^T, valid
    only without RoPE.
    """
    return Wq_head @ Bk_head.T
