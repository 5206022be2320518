"""Pins for the oracle's offline weight preparation (CPU only)."""
import numpy as np
import pytest

import synth
from oracle import prep


@pytest.fixture(scope="module")
def tiny():
    return synth.palu_tiny(seed=1)


def test_eckart_young_closed_form(tiny):
    """Truncated SVD error of W = U diag(s) V^T with s_i = exp(-i/24) at r = 32.

    Eckart-Young-Mirsky (PuzzleKV section 3.2): the Frobenius error is the root of
    the discarded squared singular values and the spectral error is s_32."""
    W = tiny["W_k"][0]
    A, B = prep.svd_factor(W, 32)
    err = W - A @ B
    fro = np.sqrt(np.sum(np.exp(-2.0 * np.arange(32, 128) / 24.0)))
    assert abs(np.linalg.norm(err) - fro) < 1e-12
    assert abs(np.linalg.norm(err, 2) - np.exp(-32.0 / 24.0)) < 1e-12
    # the printed closed-form values of the recipe
    assert abs(fro - 0.932059) < 5e-7
    assert abs(np.exp(-32.0 / 24.0) - 0.263597) < 5e-7


def test_svd_factor_split(tiny):
    """A = U_r sqrt(S_r), B = sqrt(S_r) V_r^T: A^T A = S_r = B B^T (Palu digest, Background)."""
    W = tiny["W_k"][1]
    A, B = prep.svd_factor(W, 32)
    s = tiny["sv"][:32]
    np.testing.assert_allclose(A.T @ A, np.diag(s), atol=1e-12)
    np.testing.assert_allclose(B @ B.T, np.diag(s), atol=1e-12)
    assert A.shape == (256, 32) and B.shape == (32, 128)


def test_svd_factor_full_rank_is_exact(tiny):
    W = tiny["W_v"][0]
    A, B = prep.svd_factor(W, 128)
    np.testing.assert_allclose(A @ B, W, atol=1e-12)


def test_no_other_rank_r_factorisation_is_better(tiny):
    W = tiny["W_k"][0]
    A, B = prep.svd_factor(W, 8)
    best = np.linalg.norm(W - A @ B)
    rng = np.random.default_rng(0)
    for _ in range(5):
        A2 = A + 1e-3 * rng.standard_normal(A.shape)
        B2 = B + 1e-3 * rng.standard_normal(B.shape)
        assert np.linalg.norm(W - A2 @ B2) > best


def test_factor_storage_ratio():
    # (m r + r n)/(m n) for the 4096 x 512 group matrix at rank 256 (Palu digest, Supplementary details)
    assert prep.factor_storage_ratio(4096, 512, 256) == (4096 * 256 + 256 * 512) / (4096 * 512)
    assert prep.factor_storage_ratio(4, 4, 4) == 2.0


def test_group_heads_order_and_glrd():
    rng = np.random.default_rng(3)
    heads = [rng.standard_normal((16, 4)) for _ in range(4)]
    groups = prep.group_heads(heads, 2)
    assert len(groups) == 2 and groups[0].shape == (16, 8)
    np.testing.assert_array_equal(groups[1][:, 4:], heads[3])
    A, B = prep.glrd_factor(groups, 8)      # full rank per group -> exact
    for g in range(2):
        np.testing.assert_allclose(A[g] @ B[g], groups[g], atol=1e-12)
    # J-LRD (one group of all heads) at the joint full rank is exact too
    Aj, Bj = prep.glrd_factor(prep.group_heads(heads, 4), 16)
    np.testing.assert_allclose(Aj[0] @ Bj[0], np.concatenate(heads, axis=1), atol=1e-12)


def test_glrd_error_between_mlrd_and_jlrd():
    """Same total latent size: joint >= grouped >= per-head in accuracy (Palu digest,
    Method details: J-LRD keeps shared components, M-LRD loses them)."""
    rng = np.random.default_rng(4)
    shared = rng.standard_normal((64, 6))
    heads = [shared @ rng.standard_normal((6, 8)) + 0.1 * rng.standard_normal((64, 8)) for _ in range(4)]
    full = np.concatenate(heads, axis=1)

    def err(s, r):
        gs = prep.group_heads(heads, s)
        A, B = prep.glrd_factor(gs, r)
        return np.linalg.norm(np.concatenate([A[g] @ B[g] for g in range(len(gs))], axis=1) - full)
    e_m, e_g, e_j = err(1, 2), err(2, 4), err(4, 8)
    assert e_j <= e_g <= e_m


def test_hadamard_orthogonal_exactly():
    R = prep.hadamard(64)
    assert np.array_equal(R @ R.T, np.eye(64))          # entries +-1/8 are dyadic
    assert np.array_equal(R, R.T)
    assert set(np.unique(R)) == {-0.125, 0.125}
    # Sylvester order: first row constant, row i flips on bit patterns
    assert np.all(R[0] == 0.125)
    assert R[1, 0] == 0.125 and R[1, 1] == -0.125


def test_fwht_butterfly_equals_matrix():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 64))
    np.testing.assert_allclose(prep.fwht(x), x @ prep.hadamard(64), atol=1e-13)


def test_hadamard_fold_preserves_product(tiny):
    """(A R)(R^T B) = A B (Palu digest, Method details)."""
    A, B = prep.svd_factor(tiny["W_k"][0], 64)
    R = prep.hadamard(64)
    Ah, Bh = prep.hadamard_fold(A, B, R)
    np.testing.assert_allclose(Ah @ Bh, A @ B, atol=1e-13)


def test_hadamard_spreads_first_coordinate_outliers(tiny):
    """SVD latents concentrate variance in the first coordinates (Palu digest, outliers);
    the fold spreads it: max/mean coordinate variance drops to ~1."""
    A, _ = prep.svd_factor(tiny["W_k"][0], 64)
    x = tiny["x"]
    h = x @ A
    hr = x @ (A @ prep.hadamard(64))
    v, vr = h.var(axis=0), hr.var(axis=0)
    assert v.max() / v.mean() > 3.0
    assert vr.max() / vr.mean() < 1.5


def test_value_fusion_identity(tiny):
    """p (H^v B^v) W^o = p H^v (B^v W^o) (Palu digest, Method details)."""
    rng = np.random.default_rng(6)
    A, B = prep.svd_factor(tiny["W_v"][0], 32)
    Hv = tiny["x"] @ A
    Bj = B[:, :64]
    Wo = tiny["W_o"][:64, :]
    p = rng.random(Hv.shape[0])
    p /= p.sum()
    lhs = (p @ (Hv @ Bj)) @ Wo
    rhs = (p @ Hv) @ prep.fuse_v_into_wo(Bj, Wo)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-14)


def test_key_fusion_identity(tiny):
    """q K^T = x_t (W^q (B^k)^T) (H^k)^T without RoPE (Palu digest, Method details)."""
    A, B = prep.svd_factor(tiny["W_k"][0], 32)
    x = tiny["x"]
    Hk = x @ A
    Bj = B[:, 64:128]                       # second head of the group
    Wq = tiny["W_q"][:, 64:128]
    xt = x[-1]
    lhs = (xt @ Wq) @ (Hk @ Bj).T
    rhs = (xt @ prep.fuse_k_into_wq(Wq, Bj)) @ Hk.T
    np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-13)
    assert prep.fuse_k_into_wq(Wq, Bj).shape == (256, 32)


def test_latent_project_full_rank_reconstructs_projection(tiny):
    """h = x A per unit; at full rank h_u B_u = x W_u, which fixes the orientation
    (row vectors, A on the right) and the unit order (Palu digest, Method details)."""
    As, Bs = prep.glrd_factor(tiny["W_k"], 128)
    h = prep.latent_project(tiny["x"], As)
    assert h.shape == (tiny["x"].shape[0], len(tiny["W_k"]), 128)
    for u, W in enumerate(tiny["W_k"]):
        np.testing.assert_allclose(h[:, u] @ Bs[u], tiny["x"] @ W, rtol=1e-9, atol=1e-11)


def test_latent_project_brute_force():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 5))
    A = rng.standard_normal((2, 5, 4))
    h = prep.latent_project(x, A)
    for t in range(3):
        for u in range(2):
            for i in range(4):
                assert abs(h[t, u, i] - sum(x[t, k] * A[u, k, i] for k in range(5))) < 1e-12
