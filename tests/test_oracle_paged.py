"""Pins for the oracle's hybrid paged cache and byte accounting (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import accounting, attn, codec, paged


def test_page_table_closed_form_matches_replay():
    for P, sink, win in [(4, 1, 2), (4, 1, 4), (32, 1, 4), (3, 2, 1)]:
        for T in range(1, 40 * P, 1 if P < 8 else 5):
            np.testing.assert_array_equal(paged.page_table(T, P, sink, win),
                                          paged.replay_page_table(T, P, sink, win), err_msg=f"{P} {T}")


def test_page_table_at_hybrid_workload():
    """T = 32768, P = 32, 1 sink + 4 window pages: pages 1..1019 factored."""
    tab = paged.page_table(32768, 32, 1, 4)
    assert len(tab) == 1024
    fac = np.nonzero(tab >= 0)[0]
    assert fac[0] == 1 and fac[-1] == 1019 and len(fac) == 1019
    assert tab[0] == -1 and list(tab[1020:]) == [-1 - paged.dense_slot(p, 1, 4) for p in range(1020, 1024)]
    # a page is factored exactly when the first token of page p + 4 arrives
    assert paged.page_table(32 * 8, 32, 1, 4)[4] < 0
    assert paged.page_table(32 * 8 + 1, 32, 1, 4)[4] >= 0
    assert paged.page_table(32 * 8 + 1, 32, 1, 4)[5] < 0


def test_storage_ratio_eq3(golden):
    g = golden("storage_ratio.json")
    assert paged.storage_ratio(g["r_k"], g["r_v"], g["P"], g["d"]) == g["expected"]
    # allocated bytes of the factors vs the dense page agree with Eq. 3
    dense = 2 * 32 * 128
    fact = (32 * 12 + 12 * 128) * 2
    assert fact / dense == g["expected"]


def test_kv_accounting_printed_values(golden):
    for c in golden("kv_accounting.json")["cases"]:
        assert accounting.kv_bytes(c["layers"], c["kv_heads"], c["head_dim"], c["tokens"],
                                   c["bytes_per_elem"]) == c["expected_bytes"]
    assert accounting.kv_bytes(64, 8, 128, 131072, 2) == 32 * 2 ** 30
    assert round(accounting.kv_bytes(32, 8, 128, 8192, 2) / 1e9, 2) == 1.07


def test_latent_bytes_of_the_workloads():
    assert accounting.latent_bytes(1, 8, 65536, 256) == 536870912
    assert accounting.latent_bytes(4, 8, 65536, 64, "int4") == 150994944
    assert accounting.latent_bytes(16, 8, 16384, 256) == 2147483648
    assert accounting.paged_bytes(8, 8, 5, 1019, 32, 128, 12, 12) == 8 * 8 * (5 * 16384 + 1019 * 7680)


def _page(seed, P=32, d=128, k=12, noise=0.05):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((P, k)) @ (rng.standard_normal((k, d)) / np.sqrt(k)) + noise * rng.standard_normal((P, d))


def test_factor_svd_is_eckart_young_optimal():
    X = _page(1)
    L, R = paged.factor_svd(X, 12)
    eps = paged.optimal_error(X, 12)
    assert abs(np.linalg.norm(X - L @ R) - eps) < 1e-10
    np.testing.assert_allclose(L.T @ L, np.eye(12), atol=1e-12)   # L = U_r
    rng = np.random.default_rng(2)
    for _ in range(5):
        L2 = L + 1e-3 * rng.standard_normal(L.shape)
        assert np.linalg.norm(X - L2 @ (np.linalg.pinv(L2) @ X)) >= eps - 1e-12


def test_gram_route_equals_truncated_svd():
    """Top eigenvectors of X X^T are the leading left singular vectors (PuzzleKV 3.3)."""
    for seed in range(4):
        X = _page(seed + 10)
        L1, R1 = paged.factor_svd(X, 12)
        L2, R2 = paged.factor_gram(X, 12)
        np.testing.assert_allclose(L2 @ R2, L1 @ R1, atol=1e-10)


def test_jacobi_route_equals_truncated_svd():
    X = _page(20)
    L1, R1 = paged.factor_svd(X, 12)
    L3, R3 = paged.factor_jacobi(X, 12)
    np.testing.assert_allclose(L3 @ R3, L1 @ R1, atol=1e-9)
    w, V, sweeps = paged.jacobi_eigh(X @ X.T)
    np.testing.assert_allclose(np.sort(w), np.linalg.eigvalsh(X @ X.T), rtol=1e-10, atol=1e-9)
    assert sweeps < 15


def test_exact_low_rank_page_reconstructs_exactly():
    X = _page(30, noise=0.0)
    L, R = paged.factor_gram(X, 12)
    assert np.linalg.norm(X - L @ R) < 1e-10 * np.linalg.norm(X)


def _hybrid_inputs(T, seed=5, Bsz=2, Hkv=2, g=2, P=8, r=3, d=16):
    rng = np.random.default_rng(seed)
    npg = paged.n_pages(T, P)
    dk = rng.standard_normal((Bsz, Hkv, T, d))
    dv = rng.standard_normal((Bsz, Hkv, T, d))
    Lk = rng.standard_normal((Bsz, Hkv, npg, P, r))
    Rk = rng.standard_normal((Bsz, Hkv, npg, r, d))
    Lv = rng.standard_normal((Bsz, Hkv, npg, P, r))
    Rv = rng.standard_normal((Bsz, Hkv, npg, r, d))
    q = rng.standard_normal((Bsz, Hkv * g, d))
    return q, dk, dv, Lk, Rk, Lv, Rv


def test_hybrid_pagelocal_equals_reconstruct():
    T = 83
    q, dk, dv, Lk, Rk, Lv, Rv = _hybrid_inputs(T)
    a = paged.hybrid_decode(q, [T, 50], dk, dv, Lk, Rk, Lv, Rv, 8, 1, 2, 2, form="pagelocal")
    b = paged.hybrid_decode(q, [T, 50], dk, dv, Lk, Rk, Lv, Rv, 8, 1, 2, 2, form="reconstruct")
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_all_dense_hybrid_equals_textbook():
    T = 40
    q, dk, dv, Lk, Rk, Lv, Rv = _hybrid_inputs(T)
    out = paged.hybrid_decode(q, [T, T], dk, dv, Lk, Rk, Lv, Rv, 8, 1, 10, 2)
    for b in range(2):
        for j in range(4):
            ref, _ = attn.softmax_attention(q[b, j], dk[b, j // 2], dv[b, j // 2], 1 / 4.0)
            np.testing.assert_allclose(out[b, j], ref, rtol=1e-12, atol=1e-13)


def test_full_rank_factored_pages_equal_dense():
    """Factoring every eligible page at r = P reproduces dense attention."""
    T, P, d = 96, 8, 16
    rng = np.random.default_rng(6)
    dk = rng.standard_normal((1, 1, T, d))
    dv = rng.standard_normal((1, 1, T, d))
    q = rng.standard_normal((1, 1, d))
    npg = T // P
    Lk = np.zeros((1, 1, npg, P, P)); Rk = np.zeros((1, 1, npg, P, d))
    Lv = np.zeros_like(Lk); Rv = np.zeros_like(Rk)
    for p in range(npg):
        Lk[0, 0, p], Rk[0, 0, p] = paged.factor_gram(dk[0, 0, p * P:(p + 1) * P], P)
        Lv[0, 0, p], Rv[0, 0, p] = paged.factor_svd(dv[0, 0, p * P:(p + 1) * P], P)
    out = paged.hybrid_decode(q, [T], dk, dv, Lk, Rk, Lv, Rv, P, 1, 2, 1)
    ref, _ = attn.softmax_attention(q[0, 0], dk[0, 0], dv[0, 0], 1 / 4.0)
    np.testing.assert_allclose(out[0, 0], ref, rtol=1e-10, atol=1e-12)


def test_synth_paged_pages_are_low_rank():
    """The hybrid workload's pages have the intended rank-12 + noise structure."""
    dense = synth.paged_dense(5, 1, 1, 64, 128)
    X = dense["k"][0, 0, :32].astype(np.float64)
    S = np.linalg.svd(X, compute_uv=False)
    assert S[11] > 5 * S[12]
    # noise singular values of a 32 x 128 N(0, 0.05^2) block lie near 0.05 (sqrt(128) +- sqrt(32))
    assert 0.05 * (np.sqrt(128) - np.sqrt(32)) * 0.8 < S[12:].min()
    assert S[12] < 0.05 * (np.sqrt(128) + np.sqrt(32)) * 1.2


# ----------------------------------------------------------------------------- int4 page factors

def _f16_scale(amax):
    return np.float16(np.float32(amax) / np.float32(7.0))


def test_int4_factor_groups_closed_form():
    """Each stored layout groups the elements the header documents: with F increasing
    in both indices the amax of every group is one known element, so the scales have a
    closed form, and every dequantised element sits within half its own group's scale."""
    cases = {
        # layout: (rows, cols, F[i][j], group of element (i, j), amax of group g)
        "key_L": (32, 8, lambda t, k: 1 + k + 100 * t, lambda t, k: t // 4, lambda g: 8 + 100 * (4 * g + 3)),
        "key_R": (8, 128, lambda k, d: 1 + d + 1000 * k, lambda k, d: 4 * k + d // 32,
                  lambda g: 1 + 32 * (g % 4) + 31 + 1000 * (g // 4)),
        "value_L": (32, 12, lambda t, k: 1 + t + 100 * k, lambda t, k: k, lambda g: 32 + 100 * g),
        "value_R": (12, 128, lambda k, d: 1 + d + 1000 * k, lambda k, d: 16 * (k // 4) + d // 8,
                    lambda g: 1 + 8 * (g % 16) + 7 + 1000 * (4 * (g // 16) + 3)),
    }
    for layout, (rows, cols, f, grp, amax) in cases.items():
        F = np.fromfunction(np.vectorize(f), (rows, cols), dtype=np.int64).astype(np.float64)
        codes, scales, F_hat = paged.quantize_factor(F, layout)
        n_groups = rows * cols // 32
        assert codes.shape == (rows * cols,) and scales.shape == (n_groups,)
        expect = np.array([_f16_scale(amax(g)) for g in range(n_groups)], np.float16)
        np.testing.assert_array_equal(scales, expect, err_msg=layout)
        for i in range(rows):
            for j in range(cols):
                s = float(scales[grp(i, j)])
                assert abs(F_hat[i, j] - F[i, j]) <= s / 2 + 1e-12, (layout, i, j)
        # the group's amax element is coded +-7
        assert np.all(np.max(np.abs(codes.reshape(n_groups, 32)), axis=1) == 7)


def test_int4_factor_R_formed_from_dequantised_L():
    """A page whose rows t_k = 3 + 3k are orthogonal (disjoint 8-dim supports, distinct
    norms): L = +-e_{t_k} exactly, every nonzero of L is coded 7 with scale fp16(1/7), so
    L_hat = +-c e_{t_k}, c = 7 fp16(1/7). R = L_hat^T X has rows +-c X[t_k], whose eight
    nonzeros form one group; hence X_hat row t_k = c dq(q(c X[t_k])) (sign-free, the codec
    being odd). With R taken from L instead, or L left unquantised, the result differs."""
    base = np.array([7, 2.5, -3.5, 1.5, 0.5, -6.5, 4.5, 5.5])
    X = np.zeros((32, 128))
    rows = {}
    for k in range(8):
        t = 3 + 3 * k
        X[t, 8 * k:8 * k + 8] = base * (1 + k / 4)
        rows[t] = slice(8 * k, 8 * k + 8)
    c = 7.0 * float(np.float16(np.float32(1.0) / np.float32(7.0)))

    def qdq(v):
        g = np.zeros(32, np.float32)
        g[:8] = v
        cd, sc = codec.quantize(g)
        return codec.dequantize(cd, sc)[:8].astype(np.float64)

    expect = np.zeros_like(X)
    alt = np.zeros_like(X)
    for t, sl in rows.items():
        expect[t, sl] = c * qdq(c * X[t, sl])
        alt[t, sl] = c * qdq(X[t, sl])
    assert np.any(expect != alt)
    for side in ("key", "value"):
        L_hat, R_hat, (Lc, Ls), _ = paged.factor_int4(X, 8, side)
        assert set(np.unique(np.abs(L_hat))) <= {0.0, c}
        np.testing.assert_array_equal(L_hat @ R_hat, expect, err_msg=side)


def test_int4_factor_error_bound_random_page():
    """A low-rank-plus-noise page: the int4 factors reconstruct X within the rank-r
    optimum plus the first-order effect of the two quantisation errors."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((32, 12)) @ rng.standard_normal((12, 128)) / np.sqrt(12) + 0.05 * rng.standard_normal((32, 128))
    for side in ("key", "value"):
        L_hat, R_hat, (Lc, Ls), (Rc, Rs) = paged.factor_int4(X, 12, side)
        eL = 0.5 * np.sqrt(32 * np.sum(Ls.astype(np.float64) ** 2))
        eR = 0.5 * np.sqrt(32 * np.sum(Rs.astype(np.float64) ** 2))
        bound = paged.optimal_error(X, 12) + (2 * eL + eL ** 2) * np.linalg.norm(X, 2) + (1 + eL) * eR
        assert np.linalg.norm(X - L_hat @ R_hat) <= bound
        assert np.max(np.abs(R_hat - L_hat.T @ X)) <= 0.5 * np.max(Rs.astype(np.float64)) + 1e-12
