"""GPU parity of the hybrid paged cache (append, batched page factorisation,
hybrid decode) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from oracle import attn as oattn
from oracle import paged as opaged
from tests.gpu_util import rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
P = 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as R
    R.load_library()


def _R():
    import rank_compressed_kv_amd as R
    return R


def _oracle_factors(dense, r):
    """Oracle page factors (truncated SVD) of every full page: [B][H][npg][P][r], [..][r][d]."""
    B, H, T, d = dense.shape
    npg = (T + P - 1) // P
    L = np.zeros((B, H, npg, P, r))
    Rr = np.zeros((B, H, npg, r, d))
    for b in range(B):
        for h in range(H):
            for p in range(T // P):
                L[b, h, p], Rr[b, h, p] = opaged.factor_svd(dense[b, h, p * P:(p + 1) * P].astype(np.float64), r)
    return L, Rr


def _write_cache_directly(cache, dk, dv, Lk, Rk, Lv, Rv, T):
    """Assemble a hybrid cache state of length T from given dense pages and factors
    (documented layout of include/lrkv.h): sink/window pages in their dense slots,
    every other full page as factors at slot = page."""
    B, H = dk.shape[:2]
    npg = (T + P - 1) // P
    table = np.full((B, H, cache.max_pages), -(2 ** 31), np.int32)
    dense_k = np.zeros(tuple(cache.dense_k.shape), np.float16)
    dense_v = np.zeros(tuple(cache.dense_v.shape), np.float16)
    lk = np.zeros(tuple(cache.lk.shape), np.float16)
    rk = np.zeros(tuple(cache.rk.shape), np.float16)
    lv = np.zeros(tuple(cache.lv.shape), np.float16)
    rv = np.zeros(tuple(cache.rv.shape), np.float16)
    for p in range(npg):
        lo, hi = p * P, min((p + 1) * P, T)
        if cache.sink <= p < npg - cache.window:
            table[:, :, p] = p
            lk[:, :, p], rk[:, :, p] = Lk[:, :, p], Rk[:, :, p]
            # value-side factors are stored transposed: L_V^T [r][P], R_V^T [d][r]
            lv[:, :, p], rv[:, :, p] = np.swapaxes(Lv[:, :, p], -1, -2), np.swapaxes(Rv[:, :, p], -1, -2)
        else:
            slot = p if p < cache.sink else cache.sink + (p - cache.sink) % cache.window
            table[:, :, p] = -1 - slot
            dense_k[:, :, slot, :hi - lo] = dk[:, :, lo:hi]
            dense_v[:, :, slot, :, :hi - lo] = np.swapaxes(dv[:, :, lo:hi], -1, -2)
    for name, arr in (("dense_k", dense_k), ("dense_v", dense_v), ("lk", lk), ("rk", rk), ("lv", lv),
                      ("rv", rv), ("page_table", table)):
        getattr(cache, name).copy_(torch.from_numpy(arr))
    cache.lens.fill_(T)
    cache.host_lens[:] = T


@pytest.mark.parametrize("B,H,G,T,rk,rv", [(2, 2, 4, 32 * 20 + 7, 12, 12), (1, 3, 4, 32 * 9, 12, 12),
                                            (2, 2, 2, 100, 12, 12), (1, 2, 8, 32 * 70 + 5, 12, 12),
                                            (1, 2, 16, 32 * 11 + 31, 16, 32), (2, 1, 4, 32 * 13, 20, 8)])
def test_hybrid_decode_parity(B, H, G, T, rk, rv):
    R = _R()
    say(f"hybrid decode parity: B={B} H={H} G={G} T={T} rk={rk} rv={rv}")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rv, max_pages=(T + P - 1) // P + 2)
    dense = synth.paged_dense(51, B, H, T, 128)
    npg = (T + P - 1) // P
    fk = synth.factored_pages(52, B * H * npg, P, 128, rk)
    fv = synth.factored_pages(53, B * H * npg, P, 128, rv)
    shp = lambda a, last: a.reshape((B, H, npg) + last)
    Lk, Rk = shp(fk["L"], (P, rk)), shp(fk["R"], (rk, 128))
    Lv, Rv = shp(fv["L"], (P, rv)), shp(fv["R"], (rv, 128))
    _write_cache_directly(cache, dense["k"], dense["v"], Lk, Rk, Lv, Rv, T)
    q = synth.queries(54, B, H * G, 128, 2.0)
    got = cache.decode(to_dev(q))
    torch.cuda.synchronize()
    ref = opaged.hybrid_decode(q, [T] * B, dense["k"], dense["v"], Lk, Rk, Lv, Rv, P, 1, 4, G)
    err = rel_l2(got.cpu().numpy(), ref)
    assert err.max() <= TOL, err.max()


def test_hybrid_all_dense_equals_textbook():
    """Window covering every page: the hybrid path is plain dense attention."""
    R = _R()
    B, H, G, T = 2, 2, 4, 32 * 6 - 5
    say(f"hybrid all-dense: T={T}")
    cache = R.PagedCache(B, H, G, 128, P, 1, 6, 12, 12, max_pages=8)
    dense = synth.paged_dense(55, B, H, T, 128)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    q = synth.queries(56, B, H * G, 128, 1.5)
    got = cache.decode(to_dev(q)).cpu().numpy()
    assert (cache.page_table.cpu().numpy()[:, :, :6] < 0).all()
    for b in range(B):
        for j in range(H * G):
            ref, _ = oattn.softmax_attention(q[b, j], dense["k"][b, j // G], dense["v"][b, j // G], 1 / np.sqrt(128))
            assert rel_l2(got[b, j], ref) <= TOL


@pytest.mark.parametrize("noise,rank", [(0.05, 12), (0.0, 12), (0.05, 32)])
def test_prefill_factorisation(noise, rank):
    """Prefill factors every eligible page: page table bit-exact vs the closed form,
    reconstruction error within the Eckart-Young optimum (+ fp16 storage)."""
    R = _R()
    B, H, T = 2, 2, 32 * 14 + 9
    say(f"prefill factorisation: noise={noise} rank={rank} T={T}")
    cache = R.PagedCache(B, H, 4, 128, P, 1, 4, rank, rank, max_pages=16)
    dense = synth.paged_dense(57, B, H, T, 128, noise_std=noise)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    torch.cuda.synchronize()
    table = cache.page_table.cpu().numpy()
    expect = opaged.page_table(T, P, 1, 4)
    npg = len(expect)
    assert np.array_equal(table[:, :, :npg], np.broadcast_to(expect, (B, H, npg)))
    lk, rk = cache.lk.cpu().numpy().astype(np.float64), cache.rk.cpu().numpy().astype(np.float64)
    lv = np.swapaxes(cache.lv.cpu().numpy().astype(np.float64), -1, -2)
    rv = np.swapaxes(cache.rv.cpu().numpy().astype(np.float64), -1, -2)
    for b in range(B):
        for h in range(H):
            for p in np.nonzero(expect >= 0)[0]:
                for X, L, Rm in ((dense["k"], lk, rk), (dense["v"], lv, rv)):
                    Xp = X[b, h, p * P:(p + 1) * P].astype(np.float64)
                    eps = opaged.optimal_error(Xp, rank)
                    err = np.linalg.norm(Xp - L[b, h, p] @ Rm[b, h, p])
                    assert err <= 1.01 * eps + 1e-3 * np.linalg.norm(Xp), (b, h, p, err, eps)
    # dense slots hold the sink page and the window pages
    dk = cache.dense_k.cpu().numpy()
    dv = np.swapaxes(cache.dense_v.cpu().numpy(), -1, -2)
    last = npg - 1
    slot = 1 + (last - 1) % 4
    for got, src in ((dk, dense["k"]), (dv, dense["v"])):
        assert np.array_equal(got[:, :, 0], src[:, :, :P])
        assert np.array_equal(got[:, :, slot, :T - last * P], src[:, :, last * P:T])


def test_decode_loop_against_oracle():
    """Prefill, then token-by-token appends with page factorisation as pages leave the
    window: page table bit-exact at every step, attention output against the oracle
    (which factors the same dense pages itself) at several steps."""
    R = _R()
    B, H, G = 2, 2, 4
    T0, steps = 32 * 5 + 3, 110
    say(f"decode loop: prefill {T0}, {steps} appends")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, 12, 12, max_pages=16)
    dense = synth.paged_dense(58, B, H, T0 + steps, 128)
    cache.prefill(to_dev(np.ascontiguousarray(dense["k"][:, :, :T0])),
                  to_dev(np.ascontiguousarray(dense["v"][:, :, :T0])))
    Lk, Rk = _oracle_factors(dense["k"], 12)
    Lv, Rv = _oracle_factors(dense["v"], 12)
    for i in range(steps):
        t = T0 + i
        cache.append(to_dev(np.ascontiguousarray(dense["k"][:, :, t:t + 1])),
                     to_dev(np.ascontiguousarray(dense["v"][:, :, t:t + 1])))
        T = t + 1
        tab = cache.page_table.cpu().numpy()
        expect = opaged.page_table(T, P, 1, 4)
        assert np.array_equal(tab[:, :, :len(expect)], np.broadcast_to(expect, (B, H, len(expect)))), T
        if i % 27 == 0 or i == steps - 1:
            q = synth.queries(100 + i, B, H * G, 128, 2.0)
            got = cache.decode(to_dev(q)).cpu().numpy()
            ref = opaged.hybrid_decode(q, [T] * B, dense["k"], dense["v"], Lk, Rk, Lv, Rv, P, 1, 4, G)
            assert rel_l2(got, ref).max() <= TOL, (T, rel_l2(got, ref).max())


def test_hybrid_split_independence():
    R = _R()
    B, H, G, T = 1, 2, 4, 32 * 40
    say("hybrid split independence")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, 12, 12, max_pages=48)
    dense = synth.paged_dense(59, B, H, T, 128)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    q = to_dev(synth.queries(60, B, H * G, 128, 2.0))
    outs = [cache.decode(q, n_split=n).cpu().numpy() for n in (1, 5, 40, 0)]
    # p and w = p L_V enter the value products in fp16, rounded relative to each
    # chunk's own running max, so chunkings differ by a few fp16 roundings
    for o in outs[1:]:
        assert rel_l2(o, outs[0]).max() <= 2 * 2.0 ** -11


def test_hybrid_workload_sampled():
    """Llama-3.1-8B-shaped hybrid cache at the workload's page geometry (P=32, 1 sink,
    4 window, r=12) on a reduced batch/length; sampled heads against the oracle."""
    R = _R()
    B, H, G, T = 2, 8, 4, 8192
    say(f"hybrid workload sampled: B={B} H={H} T={T}")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, 12, 12, max_pages=T // P)
    dense = synth.paged_dense(5, B, H, T, 128)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    q = synth.queries(61, B, H * G, 128, 1.0)
    got = cache.decode(to_dev(q)).cpu().numpy()
    for (b, h) in ((0, 0), (1, 5)):
        sub = lambda a: a[b:b + 1, h:h + 1]
        Lk, Rk = _oracle_factors(sub(dense["k"]), 12)
        Lv, Rv = _oracle_factors(sub(dense["v"]), 12)
        ref = opaged.hybrid_decode(q[b:b + 1, h * G:(h + 1) * G], [T], sub(dense["k"]), sub(dense["v"]),
                                   Lk, Rk, Lv, Rv, P, 1, 4, G)
        assert rel_l2(got[b, h * G:(h + 1) * G], ref[0]).max() <= TOL
