"""Hybrid paged KV cache with per-page low-rank factors, float64. Test infrastructure only.

PuzzleKV section 3.3: every layer / KV head is cut into P-token pages; a sink
page and a moving local window of recent pages stay dense, every other finished
page X (P x d) is replaced by rank-r factors X_hat = L R with L = U_r and
R = S_r W_r^T (Eq. 2). The factors come from the P x P Gram matrix X X^T: its top
r eigenvectors are the leading left singular vectors (the page's Gram route).
Decode attends over dense and factored pages together and merges the partial
results by online softmax, evaluating factored pages from their factors
(s_p = (q R^T) L^T / sqrt(d)); new tokens go to the newest dense page, and a
page is factored once it is full and has left the window (steps 4 and 5).

Readings (the pages are silent or cut off):

* page p covers tokens [p P, (p+1) P); the sink is pages [0, sink_pages); the
  window is the ``window_pages`` highest-index pages, counting the one still
  filling. With n = ceil(T / P) pages, page p is factored iff
  sink_pages <= p < n - window_pages.
* dense slots: sink page p -> slot p; other dense pages share a ring of
  ``window_pages`` slots, slot = sink_pages + (p - sink_pages) mod window_pages.
  A page leaving the window is factored before the token that reuses its slot
  is written.
* page-table entry: factored page -> p (its factor slot); dense page ->
  -1 - slot.
* the value side of a factored page (the text stops after the key-side score)
  is (a_p L^V) R^V by associativity, never forming V_hat.
* eigen-order is descending, ties broken towards the lower index.
* int4 factors (PuzzleKV, Abstract and the contributions list of section 1:
  per-factor INT4 quantisation; no grouping or order is given): each factor of a page is
  quantised with the latent codec (symmetric codes in [-7, 7], one fp16 scale
  per 32 consecutive elements) in its stored element order: keys L [P][r] and
  R [r][d] row-major, values L^T [r][P] and R^T in rank quads [r/4][d][4]. L is
  quantised first and R = L_hat^T X is formed from the dequantised L_hat, so
  that R absorbs the error of L (the least-squares R for the stored L_hat when
  L_hat has orthonormal columns).
"""
from __future__ import annotations

import math

import numpy as np

from . import codec
from .attn import chunk_partials, merge_partials


# ----------------------------------------------------------------------------- page states

def n_pages(T: int, P: int) -> int:
    return (int(T) + P - 1) // P


def is_factored(p: int, T: int, P: int, sink_pages: int, window_pages: int) -> bool:
    return sink_pages <= p < n_pages(T, P) - window_pages


def dense_slot(p: int, sink_pages: int, window_pages: int) -> int:
    return p if p < sink_pages else sink_pages + (p - sink_pages) % window_pages


def page_table(T: int, P: int, sink_pages: int, window_pages: int) -> np.ndarray:
    """Closed-form page-table entries for the ceil(T/P) pages of a length-T sequence."""
    n = n_pages(T, P)
    out = np.empty(n, dtype=np.int32)
    for p in range(n):
        if is_factored(p, T, P, sink_pages, window_pages):
            out[p] = p
        else:
            out[p] = -1 - dense_slot(p, sink_pages, window_pages)
    return out


def replay_page_table(T: int, P: int, sink_pages: int, window_pages: int) -> np.ndarray:
    """Token-by-token replay of the decode loop: each token is appended to the newest
    dense page; when a token opens a new page, the page pushed out of the window is
    factored first (its dense slot is about to be reused)."""
    table: dict[int, int] = {}
    slot_owner: dict[int, int] = {}
    for t in range(int(T)):
        if t % P == 0:
            p = t // P
            leaving = p - window_pages
            if leaving >= sink_pages:
                assert table[leaving] < 0, "a page leaves the window twice"
                table[leaving] = leaving                 # factored
                del slot_owner[dense_slot(leaving, sink_pages, window_pages)]
            slot = dense_slot(p, sink_pages, window_pages)
            assert slot not in slot_owner, "dense slot still owned by an unfactored page"
            slot_owner[slot] = p
            table[p] = -1 - slot
    return np.array([table[p] for p in range(len(table))], dtype=np.int32)


def storage_ratio(r_k: int, r_v: int, P: int, d: int) -> float:
    """rho_page = (r_K + r_V)(P + d) / (2 P d) (PuzzleKV section 3.3, Eq. 3)."""
    return (r_k + r_v) * (P + d) / (2.0 * P * d)


# ----------------------------------------------------------------------------- factorisation

def factor_svd(X: np.ndarray, r: int) -> tuple[np.ndarray, np.ndarray]:
    """Truncated SVD factors of one page: L = U_r, R = S_r W_r^T (Eq. 2)."""
    U, S, Wt = np.linalg.svd(np.asarray(X, np.float64), full_matrices=False)
    return U[:, :r], S[:r, None] * Wt[:r, :]


def optimal_error(X: np.ndarray, r: int) -> float:
    """min ||X - X_hat||_F over rank-r X_hat = sqrt(sum of the discarded S_i^2)
    (Eckart-Young-Mirsky, PuzzleKV section 3.2)."""
    S = np.linalg.svd(np.asarray(X, np.float64), compute_uv=False)
    return float(np.sqrt(np.sum(S[r:] ** 2)))


def _top_eigvecs(w: np.ndarray, V: np.ndarray, r: int) -> np.ndarray:
    order = sorted(range(len(w)), key=lambda i: (-w[i], i))
    return V[:, order[:r]]


def factor_gram(X: np.ndarray, r: int) -> tuple[np.ndarray, np.ndarray]:
    """Gram route: G = X X^T, L = top-r eigenvectors Q_r of G, R = Q_r^T X."""
    X = np.asarray(X, np.float64)
    w, V = np.linalg.eigh(X @ X.T)
    Q = _top_eigvecs(w, V, r)
    return Q, Q.T @ X


def jacobi_eigh(G: np.ndarray, tol: float = 1e-14, max_sweeps: int = 30):
    """Cyclic Jacobi eigensolver for a symmetric matrix (float64, row-cyclic order).

    Each rotation zeroes G[p, q] with t = sign(tau) / (|tau| + sqrt(1 + tau^2)),
    tau = (G[q,q] - G[p,p]) / (2 G[p,q]), c = 1/sqrt(1+t^2), s = t c.
    Stops when every |G[p,q]| <= tol * trace(|G|) or after max_sweeps sweeps.
    Returns (eigenvalues, eigenvectors as columns, sweeps used)."""
    A = np.array(G, dtype=np.float64, copy=True)
    n = A.shape[0]
    V = np.eye(n)
    scale = float(np.sum(np.abs(np.diag(A)))) or 1.0
    sweeps = 0
    for sweeps in range(1, max_sweeps + 1):
        rotated = False
        for p in range(n - 1):
            for q in range(p + 1, n):
                apq = A[p, q]
                if abs(apq) <= tol * scale:
                    continue
                rotated = True
                tau = (A[q, q] - A[p, p]) / (2.0 * apq)
                t = math.copysign(1.0, tau) / (abs(tau) + math.sqrt(1.0 + tau * tau))
                c = 1.0 / math.sqrt(1.0 + t * t)
                s = t * c
                J = np.eye(n)
                J[p, p] = c
                J[q, q] = c
                J[p, q] = s
                J[q, p] = -s
                A = J.T @ A @ J
                V = V @ J
        if not rotated:
            break
    return np.diag(A).copy(), V, sweeps


def factor_jacobi(X: np.ndarray, r: int, tol: float = 1e-14, max_sweeps: int = 30):
    """Gram route with the eigenvectors from cyclic Jacobi instead of LAPACK."""
    X = np.asarray(X, np.float64)
    w, V, _ = jacobi_eigh(X @ X.T, tol, max_sweeps)
    Q = _top_eigvecs(w, V, r)
    return Q, Q.T @ X


# ----------------------------------------------------------------------------- int4 factors

FACTOR_LAYOUTS = ("key_L", "key_R", "value_L", "value_R")


def stored_index(layout: str, rows: int, cols: int) -> np.ndarray:
    """idx with stored[e] = F.flat[idx[e]] for the logical factor F [rows][cols]
    (L [P][r] or R [r][d]) in the stored element order of ``layout``."""
    e = np.arange(rows * cols)
    if layout in ("key_L", "key_R"):
        return e                                        # row-major as is
    if layout == "value_L":                             # L^T [r][P]: e = k P + t
        k, t = e // rows, e % rows
        return t * cols + k
    if layout == "value_R":                             # rank quads: e = (k/4) 4d + 4 dim + k%4
        if rows % 4:
            raise ValueError("value R needs a rank that is a multiple of 4")
        k = 4 * (e // (4 * cols)) + e % 4
        dim = (e // 4) % cols
        return k * cols + dim
    raise ValueError(layout)


def quantize_factor(F: np.ndarray, layout: str):
    """Quantise one page factor F (logical shape) in its stored order.
    -> (codes int8 [n] in stored order, scales float16 [n/32], F_hat float64 logical)."""
    F = np.asarray(F)
    idx = stored_index(layout, *F.shape)
    codes, scales = codec.quantize(F.astype(np.float32).reshape(-1)[idx])
    F_hat = np.empty(F.size)
    F_hat[idx] = codec.dequantize(codes, scales).astype(np.float64)
    return codes, scales, F_hat.reshape(F.shape)


def factor_int4(X: np.ndarray, r: int, side: str):
    """int4 factors of one page (``side`` "key" or "value"): L from the Gram route,
    quantised; R = L_hat^T X, quantised. -> (L_hat, R_hat, (L codes, L scales),
    (R codes, R scales)), codes in stored order."""
    X = np.asarray(X, np.float64)
    L, _ = factor_gram(X, r)
    Lc, Ls, L_hat = quantize_factor(L, side + "_L")
    Rc, Rs, R_hat = quantize_factor(L_hat.T @ X, side + "_R")
    return L_hat, R_hat, (Lc, Ls), (Rc, Rs)


# ----------------------------------------------------------------------------- attention

def hybrid_attend(q: np.ndarray, pages: list, scale: float, form: str = "pagelocal") -> np.ndarray:
    """Single-query attention over a list of pages.

    ``pages`` entries are ("dense", K [n][d], V [n][d]) or
    ("factored", Lk [n][rk], Rk [rk][d], Lv [n][rv], Rv [rv][d]).
    form "reconstruct": form every factored page as L R, concatenate, textbook attention.
    form "pagelocal": score each factored page as (q R_K^T) L_K^T, value as
    (a L_V) R_V, merge per-page partial states by online softmax.
    """
    q = np.asarray(q, np.float64)
    if form == "reconstruct":
        Ks, Vs = [], []
        for pg in pages:
            if pg[0] == "dense":
                Ks.append(np.asarray(pg[1], np.float64))
                Vs.append(np.asarray(pg[2], np.float64))
            else:
                Lk, Rk, Lv, Rv = (np.asarray(a, np.float64) for a in pg[1:])
                Ks.append(Lk @ Rk)
                Vs.append(Lv @ Rv)
        K = np.concatenate(Ks)
        V = np.concatenate(Vs)
        s = (K @ q) * scale
        m = np.max(s)
        e = np.exp(s - m)
        return (e / e.sum()) @ V
    parts = []
    for pg in pages:
        if pg[0] == "dense":
            K = np.asarray(pg[1], np.float64)
            V = np.asarray(pg[2], np.float64)
            s = (K @ q) * scale
            parts.extend(chunk_partials(s, V, [(0, len(s))]))
        else:
            Lk, Rk, Lv, Rv = (np.asarray(a, np.float64) for a in pg[1:])
            s = ((q @ Rk.T) @ Lk.T) * scale
            m = np.max(s)
            a = np.exp(s - m)
            parts.append((m, np.sum(a), (a @ Lv) @ Rv))
    return merge_partials(parts)


def hybrid_decode(q, lens, dense_k, dense_v, Lk, Rk, Lv, Rv, P: int, sink_pages: int,
                  window_pages: int, g_q: int, scale=None, form: str = "pagelocal") -> np.ndarray:
    """Batch hybrid decode. q [B][Hq][d]; dense_k/v [B][Hkv][Tmax][d] hold every token at
    its position (only rows of dense pages are read); Lk/Lv [B][Hkv][pages][P][r],
    Rk/Rv [B][Hkv][pages][r][d] hold the factors of every page (only factored pages are
    read). Page states follow the closed form of ``page_table``. -> out [B][Hq][d]."""
    q = np.asarray(q, np.float64)
    Bsz, Hq, d = q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((Bsz, Hq, d))
    for b in range(Bsz):
        T = int(lens[b])
        for j in range(Hq):
            h = j // g_q
            pages = []
            for p in range(n_pages(T, P)):
                lo, hi = p * P, min((p + 1) * P, T)
                if is_factored(p, T, P, sink_pages, window_pages):
                    pages.append(("factored", Lk[b, h, p], Rk[b, h, p], Lv[b, h, p], Rv[b, h, p]))
                else:
                    pages.append(("dense", dense_k[b, h, lo:hi], dense_v[b, h, lo:hi]))
            out[b, j] = hybrid_attend(q[b, j], pages, scale, form)
    return out
