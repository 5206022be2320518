"""Pins for the oracle's decode attention (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import attn, brute, prep, rope


def _layer_dense_vs_factored(tiny, r):
    """Return (dense layer output, factored layer output) for the last token of the tiny
    layer. Dense: K = x W_k, V = x W_v per head, RoPE, textbook attention, sum_j a_j W^o_j.
    Factored: h = x A, latent-space decode, sum_j o_j (B^v_j W^o_j)."""
    x = tiny["x"]
    T = x.shape[0]
    d_h, s, nh = tiny["d_h"], tiny["s"], tiny["n_heads"]
    G = nh // s
    theta = 1e4
    q = (x[-1] @ tiny["W_q"]).reshape(nh, d_h)
    dense = np.zeros(tiny["d_model"])
    for j in range(nh):
        g, w = divmod(j, s)
        K = x @ tiny["W_k"][g][:, w * d_h:(w + 1) * d_h]
        V = x @ tiny["W_v"][g][:, w * d_h:(w + 1) * d_h]
        a, _ = attn.softmax_attention(rope.rope(q[j], T - 1, theta), rope.rope(K, np.arange(T), theta),
                                      V, 1 / np.sqrt(d_h))
        dense += a @ tiny["W_o"][j * d_h:(j + 1) * d_h]
    Ak, Bk = prep.glrd_factor(list(tiny["W_k"]), r)
    Av, Bv = prep.glrd_factor(list(tiny["W_v"]), r)
    hk = np.stack([x @ Ak[g] for g in range(G)])[None]
    hv = np.stack([x @ Av[g] for g in range(G)])[None]
    out = attn.palu_decode(hk, hv, Bk, q[None], [T], s, 1, d_h, theta)
    BvWo = np.stack([prep.fuse_v_into_wo(Bv[j // s][:, (j % s) * d_h:(j % s + 1) * d_h],
                                         tiny["W_o"][j * d_h:(j + 1) * d_h]) for j in range(nh)])
    return dense, attn.layer_output_fused(out[0], BvWo)


@pytest.fixture(scope="module")
def tiny():
    return synth.palu_tiny(seed=1)


def test_full_rank_equals_uncompressed_attention(tiny):
    """At full rank (r = s d_h = 128) the factored decode equals dense attention."""
    dense, fact = _layer_dense_vs_factored(tiny, 128)
    np.testing.assert_allclose(fact, dense, rtol=1e-10, atol=1e-12)


def test_rank32_error_is_small_but_nonzero(tiny):
    dense, fact = _layer_dense_vs_factored(tiny, 32)
    rel = np.linalg.norm(fact - dense) / np.linalg.norm(dense)
    assert 1e-6 < rel < 0.5


def test_value_fusion_at_decode_level(tiny):
    """Fused output sum_j o_j (B^v_j W^o_j) equals the unfused (p H^v B^v) W^o."""
    x = tiny["x"]
    T, d_h, s = x.shape[0], tiny["d_h"], tiny["s"]
    Ak, Bk = prep.glrd_factor(list(tiny["W_k"]), 32)
    Av, Bv = prep.glrd_factor(list(tiny["W_v"]), 32)
    hk = np.stack([x @ Ak[g] for g in range(2)])[None]
    hv = np.stack([x @ Av[g] for g in range(2)])[None]
    q = (x[-1] @ tiny["W_q"]).reshape(4, d_h)[None]
    out, probs = attn.palu_decode(hk, hv, Bk, q, [T], s, 1, d_h, 1e4, return_probs=True)
    Wo = [tiny["W_o"][j * d_h:(j + 1) * d_h] for j in range(4)]
    Bvj = [Bv[j // s][:, (j % s) * d_h:(j % s + 1) * d_h] for j in range(4)]
    fused = attn.layer_output_fused(out[0], np.stack([Bvj[j] @ Wo[j] for j in range(4)]))
    unfused = attn.layer_output_unfused([probs[(0, j)] for j in range(4)], [hv[0, j // s] for j in range(4)],
                                        Bvj, Wo)
    np.testing.assert_allclose(fused, unfused, rtol=1e-12, atol=1e-13)


def test_brute_force_tiny_shapes():
    rng = np.random.default_rng(7)
    for (T, r, d_h, s, g_q) in [(1, 4, 8, 1, 1), (5, 4, 8, 2, 1), (8, 2, 4, 1, 2), (7, 4, 6, 2, 2)]:
        U = 2
        hk = rng.standard_normal((1, U, T, r))
        hv = rng.standard_normal((1, U, T, r))
        Bk = rng.standard_normal((U, r, s * d_h))
        Hq = U * s * g_q
        q = rng.standard_normal((1, Hq, d_h))
        out = attn.palu_decode(hk, hv, Bk, q, [T], s, g_q, d_h, 1e4)
        for j in range(Hq):
            kv = j // g_q
            u, w = kv // s, kv % s
            ref = brute.palu_decode_one(hk[0, u].tolist(), hv[0, u].tolist(), Bk[u].tolist(),
                                        q[0, j].tolist(), w * d_h, d_h, 1e4, T - 1, 1 / np.sqrt(d_h))
            np.testing.assert_allclose(out[0, j], ref, rtol=1e-12, atol=1e-13)


def test_absorbed_equals_reconstruct_without_rope():
    """Key fusion at decode level: with RoPE off, H^k (q B^T) gives the same output as
    reconstructing K = H^k B."""
    rng = np.random.default_rng(8)
    U, T, r, d_h, s = 2, 40, 16, 8, 2
    hk = rng.standard_normal((2, U, T, r))
    hv = rng.standard_normal((2, U, T, r))
    Bk = rng.standard_normal((U, r, s * d_h))
    q = rng.standard_normal((2, U * s, d_h))
    qa = np.stack([[q[b, j] @ Bk[j // s][:, (j % s) * d_h:(j % s + 1) * d_h].T for j in range(U * s)]
                   for b in range(2)])
    lens = [T, 17]
    a = attn.palu_decode(hk, hv, Bk, q, lens, s, 1, d_h, 0.0)
    b = attn.palu_decode_absorbed(hk, hv, qa, lens, s, 1, d_h)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_query_position_convention():
    """q_pos defaults to len - 1, and only the relative position matters."""
    rng = np.random.default_rng(9)
    hk = rng.standard_normal((1, 1, 12, 4))
    hv = rng.standard_normal((1, 1, 12, 4))
    Bk = rng.standard_normal((1, 4, 8))
    q = rng.standard_normal((1, 1, 8))
    a = attn.palu_decode(hk, hv, Bk, q, [12], 1, 1, 8, 1e4)
    b = attn.palu_decode(hk, hv, Bk, q, [12], 1, 1, 8, 1e4, q_pos=[11])
    c = attn.palu_decode(hk, hv, Bk, q, [12], 1, 1, 8, 1e4, q_pos=[3])
    np.testing.assert_array_equal(a, b)
    assert np.abs(a - c).max() > 1e-6


def test_chunked_online_softmax_is_chunk_independent():
    rng = np.random.default_rng(10)
    T = 300
    s = rng.standard_normal(T) * 4
    V = rng.standard_normal((T, 5))
    p = np.exp(s - s.max())
    ref = (p / p.sum()) @ V
    for bounds in ([(0, T)], [(0, 1), (1, T)], [(i, min(i + 32, T)) for i in range(0, T, 32)],
                   [(0, 100), (100, 100), (100, 299), (299, 300), (300, 300)]):
        got = attn.merge_partials(attn.chunk_partials(s, V, bounds))
        np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-14)


def test_stored_formats():
    h = np.array([[1.0 / 3.0, 70000.0, -1e-9]], np.float32)
    assert attn.stored_fp16(h)[0, 0] == float(np.float16(1.0 / 3.0))
    assert np.isinf(attn.stored_fp16(h)[0, 1])
    x = np.linspace(-3, 3, 64, dtype=np.float32)[None]
    assert np.abs(attn.stored_int4(x) - x).max() <= 3 / 7 / 2 + 1e-3


def test_layer_output_fused_equals_unfused():
    """sum_j o_j (B^v_j W^o_j) = sum_j (p_j H^v B^v_j) W^o_j: the fused output projection
    the GPU path uses gives the unfused layer output (Palu digest, Method details)."""
    rng = np.random.default_rng(8)
    Hq, T, r, dh, d = 4, 9, 6, 5, 7
    Hv = rng.standard_normal((T, r))
    ps = [rng.dirichlet(np.ones(T)) for _ in range(Hq)]
    Bv = [rng.standard_normal((r, dh)) for _ in range(Hq)]
    Wo = [rng.standard_normal((dh, d)) for _ in range(Hq)]
    o = np.stack([p @ Hv for p in ps])
    fused = np.stack([prep.fuse_v_into_wo(b, w) for b, w in zip(Bv, Wo)])
    got = attn.layer_output_fused(o, fused)
    want = attn.layer_output_unfused(ps, [Hv] * Hq, Bv, Wo)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_prefill_rows_equal_decode_at_each_length():
    """Row m of a prefill chunk is one decode step at length p0 + m + 1 (causal reading);
    an off-by-one in the mask or the query position fails it."""
    rng = np.random.default_rng(21)
    B, U, s, g_q, d_h, r, T, M = 2, 2, 2, 1, 16, 8, 40, 6
    hk = rng.standard_normal((B, U, T, r))
    hv = rng.standard_normal((B, U, T, r))
    Bk = rng.standard_normal((U, r, s * d_h)) / 3
    q = rng.standard_normal((B, M, U * s * g_q, d_h))
    p0 = [T - M, 17]
    out = attn.palu_prefill(hk, hv, Bk, q, p0, s, g_q, d_h, 1e4)
    for m in range(M):
        lens = [p0[0] + m + 1, p0[1] + m + 1]
        ref = attn.palu_decode(hk, hv, Bk, q[:, m], lens, s, g_q, d_h, 1e4)
        np.testing.assert_allclose(out[:, m], ref, rtol=1e-12, atol=1e-12)


def test_prefill_is_causal_and_brute_force():
    """Tokens after a query's position do not change its row; a tiny case against the
    pure-Python loops."""
    rng = np.random.default_rng(22)
    B, U, s, g_q, d_h, r, T, M = 1, 1, 1, 2, 8, 4, 12, 4
    hk = rng.standard_normal((B, U, T, r))
    hv = rng.standard_normal((B, U, T, r))
    Bk = rng.standard_normal((U, r, s * d_h))
    q = rng.standard_normal((B, M, 2, d_h))
    p0 = [T - M]
    out = attn.palu_prefill(hk, hv, Bk, q, p0, s, g_q, d_h, 100.0)
    hk2, hv2 = hk.copy(), hv.copy()
    hk2[:, :, T - 1] += 5.0
    hv2[:, :, T - 1] -= 3.0
    out2 = attn.palu_prefill(hk2, hv2, Bk, q, p0, s, g_q, d_h, 100.0)
    np.testing.assert_allclose(out[:, :M - 1], out2[:, :M - 1], rtol=0, atol=0)
    assert np.abs(out[:, M - 1] - out2[:, M - 1]).max() > 1e-3
    for m in range(M):
        n = p0[0] + m + 1
        for j in range(2):
            ref = brute.palu_decode_one(hk[0, 0, :n].tolist(), hv[0, 0, :n].tolist(), Bk[0].tolist(),
                                        q[0, m, j].tolist(), 0, d_h, 100.0, n - 1, 1 / np.sqrt(d_h))
            np.testing.assert_allclose(out[0, m, j], ref, rtol=1e-10, atol=1e-12)
