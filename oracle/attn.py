"""Decode attention over a low-rank latent cache, float64. Test infrastructure only.

Definitions written out plainly:

* textbook attention: p = softmax(q K^T * scale), a = p V
  (Palu digest, Background: MHA; PuzzleKV section 3.2, Eq. (1)).
* reconstruct-with-RoPE path: K = H^k B^k rebuilt for every cached token,
  RoPE applied to K at each token's position and to q at the query position,
  then textbook attention against the latent values; the output stays in latent
  space, o = p H^v, because B^v is folded into W^o offline
  (Palu digest, Method details: G-LRD reconstruction, value fusion, RoPE).
* absorbed-query path (no RoPE): scores = H^k q' with q' = q (B^k)^T
  (Palu digest, Method details: key fusion).
* chunked prefill: a chunk of new tokens is appended, then each of its queries
  attends causally over the cache up to its own position (the multi-query form
  of the reconstruct-with-RoPE path; the pages describe the prefill workflow
  but print no prefill kernel, so this is the plain causal reading).

Layout and indexing readings (the pages are silent):

* Head j of ``Hq`` query heads uses KV head ``j // g_q``; KV head ``k`` lives in
  unit ``k // s`` (groups of s consecutive heads) and uses columns
  ``[(k % s) d_h, (k % s + 1) d_h)`` of that unit's B^k.
* Token t of the cache sits at position t. Decode appends first and then
  attends, so the query position defaults to ``len - 1``.
* The softmax scale defaults to 1/sqrt(d_h) on both paths (also in the absorbed
  path, whose contraction length is r).
"""
from __future__ import annotations

import numpy as np

from . import codec
from .rope import rope


def softmax_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Single-query attention. q [d], K [T][d], V [T][e] -> (a [e], p [T])."""
    s = (np.asarray(K, np.float64) @ np.asarray(q, np.float64)) * scale
    m = np.max(s)
    e = np.exp(s - m)
    p = e / np.sum(e)
    return p @ np.asarray(V, np.float64), p


def head_unit(j: int, s: int, g_q: int) -> tuple[int, int]:
    """(unit, head-within-unit) of the KV head serving query head j."""
    k = j // g_q
    return k // s, k % s


def stored_fp16(h: np.ndarray) -> np.ndarray:
    """Latents as the fp16 cache holds them: round-to-nearest-even to fp16, read back exactly."""
    with np.errstate(over="ignore"):
        return np.asarray(h, np.float32).astype(np.float16).astype(np.float64)


def stored_int4(h: np.ndarray) -> np.ndarray:
    """Latents as the int4 cache holds them: quantise per 32-group, dequantise exactly."""
    codes, scales = codec.quantize(np.asarray(h, np.float32))
    return codec.dequantize(codes, scales).astype(np.float64)


def palu_decode(hk, hv, Bk, q, lens, s: int, g_q: int, d_h: int, theta: float,
                q_pos=None, sm_scale=None, return_probs: bool = False):
    """Reconstruct-with-RoPE decode attention, latent-space output.

    hk, hv [B][U][T][r] stored latent values (already decoded to float), Bk
    [U][r][s*d_h], q [B][Hq][d_h] un-rotated queries, lens [B] -> out [B][Hq][r].
    theta == 0 disables RoPE.
    """
    hk = np.asarray(hk, np.float64)
    hv = np.asarray(hv, np.float64)
    Bk = np.asarray(Bk, np.float64)
    q = np.asarray(q, np.float64)
    Bsz, Hq = q.shape[0], q.shape[1]
    r = hk.shape[-1]
    scale = 1.0 / np.sqrt(d_h) if sm_scale is None else sm_scale
    out = np.zeros((Bsz, Hq, r))
    probs = {}
    for b in range(Bsz):
        T = int(lens[b])
        qp = T - 1 if q_pos is None else int(q_pos[b])
        pos = np.arange(T)
        for j in range(Hq):
            u, w = head_unit(j, s, g_q)
            K = hk[b, u, :T] @ Bk[u][:, w * d_h:(w + 1) * d_h]        # reconstruction
            Kr = rope(K, pos, theta)
            qr = rope(q[b, j], qp, theta)
            out[b, j], p = softmax_attention(qr, Kr, hv[b, u, :T], scale)
            probs[(b, j)] = p
    return (out, probs) if return_probs else out


def palu_prefill(hk, hv, Bk, q, p0, s: int, g_q: int, d_h: int, theta: float, sm_scale=None):
    """Chunked-prefill (multi-query) attention on the reconstruct-with-RoPE path.

    The M new tokens of sequence b sit at positions p0[b] .. p0[b] + M - 1 of the
    cache (appended before the call); query m attends causally, to tokens
    0 .. p0[b] + m, exactly as one decode step at that length would (same
    reconstruction, RoPE at each side's position, latent-space output).
    hk, hv [B][U][T][r], Bk [U][r][s*d_h], q [B][M][Hq][d_h], p0 [B] ->
    out [B][M][Hq][r].
    """
    hk = np.asarray(hk, np.float64)
    hv = np.asarray(hv, np.float64)
    Bk = np.asarray(Bk, np.float64)
    q = np.asarray(q, np.float64)
    Bsz, M, Hq = q.shape[0], q.shape[1], q.shape[2]
    r = hk.shape[-1]
    scale = 1.0 / np.sqrt(d_h) if sm_scale is None else sm_scale
    out = np.zeros((Bsz, M, Hq, r))
    for b in range(Bsz):
        T = int(p0[b]) + M
        pos = np.arange(T)
        for j in range(Hq):
            u, w = head_unit(j, s, g_q)
            Kr = rope(hk[b, u, :T] @ Bk[u][:, w * d_h:(w + 1) * d_h], pos, theta)
            for m in range(M):
                n = int(p0[b]) + m + 1                                   # causal: tokens < n
                qr = rope(q[b, m, j], n - 1, theta)
                out[b, m, j], _ = softmax_attention(qr, Kr[:n], hv[b, u, :n], scale)
    return out


def palu_decode_absorbed(hk, hv, qa, lens, s: int, g_q: int, d_h: int, sm_scale=None):
    """Absorbed-query decode attention (no RoPE): scores = H^k q'_j * scale.

    qa [B][Hq][r] absorbed queries q'_j = q_j (B^k_j)^T -> out [B][Hq][r].
    """
    hk = np.asarray(hk, np.float64)
    hv = np.asarray(hv, np.float64)
    qa = np.asarray(qa, np.float64)
    Bsz, Hq, r = qa.shape
    scale = 1.0 / np.sqrt(d_h) if sm_scale is None else sm_scale
    out = np.zeros((Bsz, Hq, r))
    for b in range(Bsz):
        T = int(lens[b])
        for j in range(Hq):
            u, _ = head_unit(j, s, g_q)
            out[b, j], _ = softmax_attention(qa[b, j], hk[b, u, :T], hv[b, u, :T], scale)
    return out


def chunk_partials(scores: np.ndarray, V: np.ndarray, bounds: list[tuple[int, int]]):
    """Per-chunk softmax state (m, l, acc) of already-scaled scores [T] against V [T][e].
    An empty chunk gives (-inf, 0, 0)."""
    parts = []
    for lo, hi in bounds:
        if hi <= lo:
            parts.append((-np.inf, 0.0, np.zeros(V.shape[-1])))
            continue
        sc = scores[lo:hi]
        m = np.max(sc)
        e = np.exp(sc - m)
        parts.append((m, np.sum(e), e @ V[lo:hi]))
    return parts


def merge_partials(parts) -> np.ndarray:
    """Online-softmax merge of chunk states: m = max m_c,
    o = sum_c e^{m_c - m} acc_c / sum_c e^{m_c - m} l_c; empty chunks contribute nothing.
    (PuzzleKV section 3.3, step 4: partial results merged by online softmax.)"""
    ms = np.array([p[0] for p in parts])
    m = np.max(ms)
    w = np.where(np.isfinite(ms), np.exp(ms - m), 0.0)
    num = sum(wc * p[2] for wc, p in zip(w, parts))
    den = sum(wc * p[1] for wc, p in zip(w, parts))
    return num / den


def layer_output_fused(out_latent: np.ndarray, BvWo: np.ndarray) -> np.ndarray:
    """sum_j o_j (B^v_j W^o_j): out_latent [Hq][r], BvWo [Hq][r][d] -> [d]."""
    return np.einsum("jr,jrd->d", np.asarray(out_latent, np.float64), np.asarray(BvWo, np.float64))


def layer_output_unfused(p_list, Hv_list, Bv_list, Wo_list) -> np.ndarray:
    """sum_j (p_j H^v_j B^v_j) W^o_j: the value reconstructed explicitly, then projected."""
    return sum((p @ Hv @ Bv) @ Wo for p, Hv, Bv, Wo in zip(p_list, Hv_list, Bv_list, Wo_list))
