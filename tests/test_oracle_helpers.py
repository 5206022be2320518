"""Direct pins of the oracle's small helpers (each is also exercised through the
functions that use them): head-to-unit mapping, rotate-half, the factored-page
predicate and the stored orders of int4 page factors."""
import numpy as np
import pytest

from oracle import attn, paged, rope


def test_head_unit_closed_form():
    # G-LRD units of s = 4 heads, no GQA (the Llama-2-7B layer): head j -> (j // 4, j % 4)
    assert [attn.head_unit(j, 4, 1) for j in range(8)] == [(0, 0), (0, 1), (0, 2), (0, 3),
                                                          (1, 0), (1, 1), (1, 2), (1, 3)]
    # one KV head per unit shared by 4 query heads (Llama-3-8B GQA): j -> (j // 4, 0)
    assert [attn.head_unit(j, 1, 4) for j in range(8)] == [(0, 0)] * 4 + [(1, 0)] * 4
    # s = 2 KV heads per unit, 2 query heads each: KV head j // 2, unit (j // 2) // 2
    assert [attn.head_unit(j, 2, 2) for j in range(8)] == [(0, 0), (0, 0), (0, 1), (0, 1),
                                                          (1, 0), (1, 0), (1, 1), (1, 1)]


def test_rotate_half():
    x = np.array([1.0, 2.0, 3.0, 4.0])
    assert np.array_equal(rope.rotate_half(x), np.array([-3.0, -4.0, 1.0, 2.0]))
    y = np.random.default_rng(0).standard_normal((3, 8))
    assert np.array_equal(rope.rotate_half(rope.rotate_half(y)), -y)


@pytest.mark.parametrize("T,expect", [(320, [1, 2, 3, 4, 5]),        # 10 full pages
                                      (330, [1, 2, 3, 4, 5, 6]),     # 11 pages, last partial
                                      (160, []),                     # sink + window only
                                      (32, [])])
def test_is_factored(T, expect):
    # P = 32, one sink page, four window pages: pages 1 .. n - 5 are factored
    n = paged.n_pages(T, 32)
    assert [p for p in range(n) if paged.is_factored(p, T, 32, 1, 4)] == expect


@pytest.mark.parametrize("layout,rows,cols", [("key_L", 32, 12), ("key_R", 12, 128),
                                              ("value_L", 32, 12), ("value_R", 12, 128),
                                              ("value_R", 4, 3)])
def test_stored_index_is_a_permutation(layout, rows, cols):
    idx = paged.stored_index(layout, rows, cols)
    assert np.array_equal(np.sort(idx), np.arange(rows * cols))


def test_stored_index_orders():
    F = np.arange(32 * 12).reshape(32, 12)
    assert np.array_equal(F.flat[paged.stored_index("key_L", 32, 12)], F.reshape(-1))
    # value L is stored transposed: L^T [r][P]
    assert np.array_equal(F.flat[paged.stored_index("value_L", 32, 12)], F.T.reshape(-1))
    # value R [r][d] in rank quads: for each quad of ranks, dim-major runs of 4 ranks
    G = np.arange(4 * 3).reshape(4, 3)          # G[k][dim] = 3 k + dim
    assert list(G.flat[paged.stored_index("value_R", 4, 3)]) == [0, 3, 6, 9, 1, 4, 7, 10, 2, 5, 8, 11]
    with pytest.raises(ValueError):
        paged.stored_index("value_R", 6, 3)


def test_hybrid_attend_against_library_softmax():
    """Page-local scoring and value products over mixed dense / factored pages
    (unequal key and value ranks) equal softmax attention, by scipy, over the
    concatenation of every page's K = L R and V = L R."""
    from scipy.special import softmax
    rng = np.random.default_rng(3)
    d, P = 16, 8
    q = rng.standard_normal(d)
    pages, Ks, Vs = [], [], []
    for kind, n in (("dense", P), ("factored", P), ("dense", 5), ("factored", P)):
        if kind == "dense":
            K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
            pages.append(("dense", K, V))
        else:
            Lk, Rk = rng.standard_normal((n, 3)), rng.standard_normal((3, d))
            Lv, Rv = rng.standard_normal((n, 2)), rng.standard_normal((2, d))
            pages.append(("factored", Lk, Rk, Lv, Rv))
            K, V = Lk @ Rk, Lv @ Rv
        Ks.append(K)
        Vs.append(V)
    scale = 0.3
    ref = softmax(np.concatenate(Ks) @ q * scale) @ np.concatenate(Vs)
    for form in ("pagelocal", "reconstruct"):
        assert np.allclose(paged.hybrid_attend(q, pages, scale, form), ref, rtol=1e-12, atol=1e-12)
