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


def _oracle(q, T, dk, dv, Lk, Rk, Lv, Rv, sink, window, G):
    """The oracle's hybrid decode in its plain form: every factored page rebuilt as
    L R, all pages concatenated, textbook softmax attention."""
    lens = [T] * q.shape[0] if np.isscalar(T) else T
    return opaged.hybrid_decode(q, lens, dk, dv, Lk, Rk, Lv, Rv, P, sink, window, G, form="reconstruct")


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
                                            (1, 2, 16, 32 * 11 + 31, 16, 32), (2, 1, 4, 32 * 13, 20, 8),
                                            (1, 2, 4, 32 * 21 + 3, 4, 4), (2, 1, 4, 32 * 17 + 9, 8, 8),
                                            (1, 2, 4, 32 * 15 + 1, 16, 16), (1, 2, 4, 32 * 12 + 5, 12, 8)])
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
    ref = _oracle(q, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
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
            ref = _oracle(q, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
            assert rel_l2(got, ref).max() <= TOL, (T, rel_l2(got, ref).max())


@pytest.mark.parametrize("T", [32 * 128, 32 * 128 + 19])
def test_hybrid_split_independence(T):
    """Every split count checked against the oracle (plain reconstruct form) and
    against each other. n_split = 1 is raised to the fewest chunks of at most 64
    pages, so one wave walks 64 pages (43 at T = 4115) and uses every bit of its
    factored / dense page masks."""
    R = _R()
    B, H, G, rk, rv = 1, 2, 4, 12, 12
    say(f"hybrid split independence: T={T}, n_split 1/5/40/auto")
    npg = (T + P - 1) // P
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rv, max_pages=npg + 2)
    dense = synth.paged_dense(59, B, H, T, 128)
    fk = synth.factored_pages(62, B * H * npg, P, 128, rk)
    fv = synth.factored_pages(63, B * H * npg, P, 128, rv)
    shp = lambda a, last: a.reshape((B, H, npg) + last)
    Lk, Rk = shp(fk["L"], (P, rk)), shp(fk["R"], (rk, 128))
    Lv, Rv = shp(fv["L"], (P, rv)), shp(fv["R"], (rv, 128))
    _write_cache_directly(cache, dense["k"], dense["v"], Lk, Rk, Lv, Rv, T)
    qh = synth.queries(60, B, H * G, 128, 2.0)
    q = to_dev(qh)
    outs = [cache.decode(q, n_split=n).cpu().numpy() for n in (1, 5, 40, 0)]
    ref = _oracle(qh, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
    for o in outs:
        assert rel_l2(o, ref).max() <= TOL, rel_l2(o, ref).max()
    # p and w = p L_V enter the value products in fp16, rounded relative to each
    # chunk's own running max, so chunkings differ by a few fp16 roundings
    for o in outs[1:]:
        assert rel_l2(o, outs[0]).max() <= 2 * 2.0 ** -11


@pytest.mark.parametrize("n_split", [0, 32])
def test_hybrid_workload_full_sampled(n_split):
    """The hybrid decode at the workload's full size (8 sequences x 8 KV heads x 32K
    tokens, P = 32, 1 sink + 4 window pages, rank 12, fp16 factors) in the launch
    configuration the benchmark times (default chunking: 16 chunks of 64 pages per
    (sequence, KV head), so each wave uses all 64 bits of its page masks), and
    with 32 chunks of 32 pages. Factors and dense pages are
    written on the device by torch from a seeded generator (L entries of size
    1/sqrt(P), R entries of size 3); sampled (sequence, KV head) pairs are read
    back and checked against the oracle's plain reconstruct form."""
    R = _R()
    B, H, G, T, rk = 8, 8, 4, 32768, 12
    say(f"hybrid workload full sampled: fp16 factors B={B} H={H} T={T} n_split={n_split}")
    dev = torch.device("cuda")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rk, max_pages=T // P + 8)
    g = torch.Generator(device=dev)
    g.manual_seed(90)
    npg = T // P
    expect = opaged.page_table(T, P, 1, 4)
    cache.page_table[:, :, :npg] = torch.from_numpy(expect).to(dev)
    cache.lens.fill_(T)
    cache.host_lens[:] = T
    for n, sd in (("lk", P ** -0.5), ("rk", 3.0), ("lv", P ** -0.5), ("rv", 3.0)):
        a = getattr(cache, n)
        a.copy_((torch.randn(a.shape, generator=g, device=dev) * sd).half())
    cache.dense_k.copy_(torch.randn(cache.dense_k.shape, generator=g, device=dev).half())
    cache.dense_v.copy_(torch.randn(cache.dense_v.shape, generator=g, device=dev).half())
    q = torch.randn((B, H * G, 128), generator=g, device=dev)
    got = cache.decode(q, n_split=n_split).cpu().numpy()
    assert np.isfinite(got).all()
    qn = q.cpu().numpy().astype(np.float64)
    for (b, h) in ((0, 0), (3, 6), (7, 7)):
        lk = cache.lk[b, h, :npg].cpu().numpy().astype(np.float64)[None, None]
        rk_ = cache.rk[b, h, :npg].cpu().numpy().astype(np.float64)[None, None]
        lv = np.swapaxes(cache.lv[b, h, :npg].cpu().numpy().astype(np.float64), -1, -2)[None, None]
        rv = np.swapaxes(cache.rv[b, h, :npg].cpu().numpy().astype(np.float64), -1, -2)[None, None]
        dk = np.zeros((1, 1, T, 128))
        dv = np.zeros((1, 1, T, 128))
        dks = cache.dense_k[b, h].cpu().numpy().astype(np.float64)
        dvs = np.swapaxes(cache.dense_v[b, h].cpu().numpy().astype(np.float64), -1, -2)
        for p in np.nonzero(expect < 0)[0]:
            slot = -1 - expect[p]
            dk[0, 0, p * P:(p + 1) * P] = dks[slot]
            dv[0, 0, p * P:(p + 1) * P] = dvs[slot]
        ref = _oracle(qn[b:b + 1, h * G:(h + 1) * G], T, dk, dv, lk, rk_, lv, rv, 1, 4, G)
        err = rel_l2(got[b, h * G:(h + 1) * G], ref[0]).max()
        say(f"  (b={b}, h={h}) max rel-L2 {err:.3g}")
        assert err <= TOL, ((b, h), err)


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
        ref = _oracle(q[b:b + 1, h * G:(h + 1) * G], T, sub(dense["k"]), sub(dense["v"]), Lk, Rk, Lv, Rv, 1, 4, G)
        assert rel_l2(got[b, h * G:(h + 1) * G], ref[0]).max() <= TOL


# ----------------------------------------------------------------------------- int4 page factors
# Stored layouts (include/lrkv.h): codes two per byte (element 2i in the low
# nibble) in each factor's stored element order, one fp16 scale per 32 elements.
# The decoding helpers below are test-side layout code; the oracle only supplies
# the element order (a function of the sizes) and the quantised inputs.

_LAYOUT_SHAPES = {"key_L": lambda r: (P, r), "key_R": lambda r: (r, 128),
                  "value_L": lambda r: (P, r), "value_R": lambda r: (r, 128)}


def _pack(codes):
    c = np.asarray(codes).astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def _unpack(b):
    b = np.asarray(b).astype(np.int16)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int16)
    out[..., 0::2], out[..., 1::2] = b & 0xF, (b >> 4) & 0xF
    return np.where(out >= 8, out - 16, out)


def _from_stored(codes_u8, scales, layout, r):
    """Stored codes [..., n/2] + scales [..., n/32] -> (logical factors float64,
    logical codes, per-element scale), for every leading index."""
    rows, cols = _LAYOUT_SHAPES[layout](r)
    idx = opaged.stored_index(layout, rows, cols)
    c = _unpack(codes_u8)
    s = np.repeat(np.asarray(scales).astype(np.float64), 32, axis=-1)
    lead = c.shape[:-1]
    F = np.empty(lead + (rows * cols,))
    C = np.empty(lead + (rows * cols,), np.int16)
    S = np.empty(lead + (rows * cols,))
    F[..., idx] = c * s
    C[..., idx] = c
    S[..., idx] = s
    sh = lead + (rows, cols)
    return F.reshape(sh), C.reshape(sh), S.reshape(sh)


def _write_int4_cache(cache, dk, dv, Lk, Rk, Lv, Rv, T):
    """As _write_cache_directly, with every factored page quantised by the oracle's
    int4 factor codec; returns the dequantised factors the oracle decodes with."""
    B, H = dk.shape[:2]
    npg = (T + P - 1) // P
    table = np.full((B, H, cache.max_pages), -(2 ** 31), np.int32)
    dense_k = np.zeros(tuple(cache.dense_k.shape), np.float16)
    dense_v = np.zeros(tuple(cache.dense_v.shape), np.float16)
    arrs = {n: np.zeros(tuple(getattr(cache, n).shape), np.uint8) for n in ("lk", "rk", "lv", "rv")}
    sc = {n: np.zeros(tuple(getattr(cache, n + "_s").shape), np.float16) for n in ("lk", "rk", "lv", "rv")}
    hat = {n: np.zeros_like(a, np.float64) for n, a in (("lk", Lk), ("rk", Rk), ("lv", Lv), ("rv", Rv))}
    src = {"lk": (Lk, "key_L"), "rk": (Rk, "key_R"), "lv": (Lv, "value_L"), "rv": (Rv, "value_R")}
    for p in range(npg):
        lo, hi = p * P, min((p + 1) * P, T)
        if cache.sink <= p < npg - cache.window:
            table[:, :, p] = p
            for b in range(B):
                for h in range(H):
                    for n, (F, layout) in src.items():
                        codes, scales, F_hat = opaged.quantize_factor(F[b, h, p], layout)
                        arrs[n][b, h, p], sc[n][b, h, p], hat[n][b, h, p] = _pack(codes), scales, F_hat
        else:
            slot = p if p < cache.sink else cache.sink + (p - cache.sink) % cache.window
            table[:, :, p] = -1 - slot
            dense_k[:, :, slot, :hi - lo] = dk[:, :, lo:hi]
            dense_v[:, :, slot, :, :hi - lo] = np.swapaxes(dv[:, :, lo:hi], -1, -2)
    cache.dense_k.copy_(torch.from_numpy(dense_k))
    cache.dense_v.copy_(torch.from_numpy(dense_v))
    cache.page_table.copy_(torch.from_numpy(table))
    for n in arrs:
        getattr(cache, n).copy_(torch.from_numpy(arrs[n]))
        getattr(cache, n + "_s").copy_(torch.from_numpy(sc[n]))
    cache.lens.fill_(T)
    cache.host_lens[:] = T
    return hat["lk"], hat["rk"], hat["lv"], hat["rv"]


@pytest.mark.parametrize("B,H,G,T,rk,rv", [(2, 2, 4, 32 * 20 + 7, 12, 12), (1, 2, 16, 32 * 11 + 31, 16, 8),
                                            (2, 1, 8, 32 * 13, 4, 16), (1, 3, 2, 100, 8, 12),
                                            (1, 2, 4, 32 * 70 + 5, 12, 12)])
def test_hybrid_int4_decode_parity(B, H, G, T, rk, rv):
    """Decode over int4 page factors against the oracle on the same dequantised factors."""
    R = _R()
    say(f"hybrid int4 decode parity: B={B} H={H} G={G} T={T} rk={rk} rv={rv}")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rv, max_pages=(T + P - 1) // P + 2,
                         factor_fmt=R.FMT_INT4_G32)
    dense = synth.paged_dense(71, B, H, T, 128)
    npg = (T + P - 1) // P
    fk = synth.factored_pages(72, B * H * npg, P, 128, rk)
    fv = synth.factored_pages(73, B * H * npg, P, 128, rv)
    shp = lambda a, last: a.reshape((B, H, npg) + last).astype(np.float64)
    Lk, Rk = shp(fk["L"], (P, rk)), shp(fk["R"], (rk, 128))
    Lv, Rv = shp(fv["L"], (P, rv)), shp(fv["R"], (rv, 128))
    Lk, Rk, Lv, Rv = _write_int4_cache(cache, dense["k"], dense["v"], Lk, Rk, Lv, Rv, T)
    q = synth.queries(74, B, H * G, 128, 2.0)
    got = cache.decode(to_dev(q))
    torch.cuda.synchronize()
    ref = _oracle(q, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
    err = rel_l2(got.cpu().numpy(), ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("noise,rank", [(0.05, 12), (0.0, 16), (0.05, 4)])
def test_prefill_factorisation_int4(noise, rank):
    """int4 factors written by prefill: page table bit-exact; codes in [-7, 7] with the
    amax element of every group with a normal scale coded +-7; R within half a scale of
    L_hat^T X (R formed from the dequantised L, then quantised) and each scale
    fp16(amax / 7) of that product; reconstruction within the rank-r optimum plus
    the first-order effect of both quantisation errors."""
    R = _R()
    B, H, T = 2, 2, 32 * 14 + 9
    say(f"prefill factorisation int4: noise={noise} rank={rank} T={T}")
    cache = R.PagedCache(B, H, 4, 128, P, 1, 4, rank, rank, max_pages=16, factor_fmt=R.FMT_INT4_G32)
    dense = synth.paged_dense(75, B, H, T, 128, noise_std=noise)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    torch.cuda.synchronize()
    table = cache.page_table.cpu().numpy()
    expect = opaged.page_table(T, P, 1, 4)
    npg = len(expect)
    assert np.array_equal(table[:, :, :npg], np.broadcast_to(expect, (B, H, npg)))
    dec = {}
    for n, layout in (("lk", "key_L"), ("rk", "key_R"), ("lv", "value_L"), ("rv", "value_R")):
        codes = getattr(cache, n).cpu().numpy()
        scales = getattr(cache, n + "_s").cpu().numpy()
        dec[n] = _from_stored(codes, scales, layout, rank)
        c = _unpack(codes)
        grp = np.abs(c.reshape(c.shape[:-1] + (-1, 32))).max(axis=-1)
        fac = expect >= 0
        s = scales[:, :, :npg][:, :, fac].astype(np.float64)
        g = grp[:, :, :npg][:, :, fac]
        assert np.all(s >= 0)
        # (a subnormal fp16 scale is coarser than amax / 7: its amax code may be below 7)
        assert np.all(g[s >= 2.0 ** -14] == 7) and np.all(g[s == 0] == 0), n
    for b in range(B):
        for h in range(H):
            for p in np.nonzero(expect >= 0)[0]:
                for X, ln, rn in ((dense["k"], "lk", "rk"), (dense["v"], "lv", "rv")):
                    Xp = X[b, h, p * P:(p + 1) * P].astype(np.float64)
                    L, _, SL = (a[b, h, p] for a in dec[ln])
                    Rm, _, SR = (a[b, h, p] for a in dec[rn])
                    LtX = L.T @ Xp
                    xmax = np.max(np.abs(Xp))
                    # R: the codec applied to L_hat^T X (accumulated in fp32 on the GPU)
                    assert np.all(np.abs(Rm - LtX) <= 0.5 * SR * (1 + 1e-3) + 1e-4 * xmax), (b, h, p, rn)
                    rs = np.unique(SR)
                    for sv in rs[rs > 0]:
                        amax = np.max(np.abs(LtX[SR == sv]))
                        assert abs(sv - amax / 7) <= 2.0 ** -11 * sv + 1e-4 * xmax, (b, h, p, rn)
                    eL = 0.5 * np.sqrt(np.sum(SL ** 2))
                    eR = 0.5 * np.sqrt(np.sum(SR ** 2))
                    bound = (1.01 * opaged.optimal_error(Xp, rank) + 1e-3 * np.linalg.norm(Xp)
                             + (2 * eL + eL ** 2) * np.linalg.norm(Xp, 2) + (1 + eL) * eR)
                    assert np.linalg.norm(Xp - L @ Rm) <= bound, (b, h, p)


def test_int4_decode_loop_end_to_end():
    """Prefill, then appends that push pages out of the window (factored from their
    dense slots): page table bit-exact; the output's distance from exact rank-r
    attention (float64 truncated SVD) is of the size of the oracle's own int4 factor
    error on the same pages."""
    R = _R()
    B, H, G, rank = 2, 2, 4, 12
    T0, steps = 32 * 12 + 5, 40
    say(f"int4 decode loop: prefill {T0}, {steps} appends")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rank, rank, max_pages=16, factor_fmt=R.FMT_INT4_G32)
    dense = synth.paged_dense(76, B, H, T0 + steps, 128)
    cache.prefill(to_dev(np.ascontiguousarray(dense["k"][:, :, :T0])),
                  to_dev(np.ascontiguousarray(dense["v"][:, :, :T0])))
    for i in range(steps):
        t = T0 + i
        cache.append(to_dev(np.ascontiguousarray(dense["k"][:, :, t:t + 1])),
                     to_dev(np.ascontiguousarray(dense["v"][:, :, t:t + 1])))
    T = T0 + steps
    expect = opaged.page_table(T, P, 1, 4)
    tab = cache.page_table.cpu().numpy()
    assert np.array_equal(tab[:, :, :len(expect)], np.broadcast_to(expect, (B, H, len(expect))))
    q = synth.queries(77, B, H * G, 128, 2.0)
    got = cache.decode(to_dev(q)).cpu().numpy()
    Lk, Rk = _oracle_factors(dense["k"][:, :, :T], rank)
    Lv, Rv = _oracle_factors(dense["v"][:, :, :T], rank)
    exact = _oracle(q, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
    q4 = [np.zeros_like(a) for a in (Lk, Rk, Lv, Rv)]
    for b in range(B):
        for h in range(H):
            for p in range(T // P):
                for X, side, i in ((dense["k"], "key", 0), (dense["v"], "value", 2)):
                    L_hat, R_hat, _, _ = opaged.factor_int4(X[b, h, p * P:(p + 1) * P], rank, side)
                    q4[i][b, h, p], q4[i + 1][b, h, p] = L_hat, R_hat
    ref4 = _oracle(q, T, dense["k"], dense["v"], *q4, 1, 4, G)
    e_oracle = rel_l2(ref4, exact).max()
    e_gpu = rel_l2(got, exact).max()
    say(f"  int4 error vs exact rank-r attention: gpu {e_gpu:.3e}, oracle {e_oracle:.3e}")
    assert e_gpu <= 2 * e_oracle + TOL, (e_gpu, e_oracle)


def test_hybrid_int4_sink_window_geometry():
    """int4 factors with 2 sink and 3 window pages, unequal ranks (8 / 4): the page
    table and dense slots follow the geometry, decode against the oracle."""
    R = _R()
    B, H, G, T, rk, rv = 2, 2, 4, 32 * 17 + 9, 8, 4
    say(f"hybrid int4 sink/window: T={T} rk={rk} rv={rv}")
    cache = R.PagedCache(B, H, G, 128, P, 2, 3, rk, rv, max_pages=(T + P - 1) // P + 1,
                         factor_fmt=R.FMT_INT4_G32)
    dense = synth.paged_dense(81, B, H, T, 128)
    npg = (T + P - 1) // P
    fk = synth.factored_pages(82, B * H * npg, P, 128, rk)
    fv = synth.factored_pages(83, B * H * npg, P, 128, rv)
    shp = lambda a, last: a.reshape((B, H, npg) + last).astype(np.float64)
    Lk, Rk = shp(fk["L"], (P, rk)), shp(fk["R"], (rk, 128))
    Lv, Rv = shp(fv["L"], (P, rv)), shp(fv["R"], (rv, 128))
    Lk, Rk, Lv, Rv = _write_int4_cache(cache, dense["k"], dense["v"], Lk, Rk, Lv, Rv, T)
    q = synth.queries(84, B, H * G, 128, 2.0)
    got = cache.decode(to_dev(q)).cpu().numpy()
    ref = _oracle(q, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 2, 3, G)
    assert rel_l2(got, ref).max() <= TOL


@pytest.mark.parametrize("T", [32 * 128, 32 * 70 + 5])
def test_hybrid_int4_split_independence(T):
    """int4 factors (oracle-quantised): every split count against the oracle and
    against each other; n_split = 1 gives one wave up to 64 pages."""
    R = _R()
    B, H, G, rk, rv = 1, 2, 4, 12, 12
    say(f"hybrid int4 split independence: T={T}, n_split 1/5/40/auto")
    npg = (T + P - 1) // P
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rv, max_pages=npg + 2, factor_fmt=R.FMT_INT4_G32)
    dense = synth.paged_dense(78, B, H, T, 128)
    fk = synth.factored_pages(85, B * H * npg, P, 128, rk)
    fv = synth.factored_pages(86, B * H * npg, P, 128, rv)
    shp = lambda a, last: a.reshape((B, H, npg) + last).astype(np.float64)
    Lk, Rk = shp(fk["L"], (P, rk)), shp(fk["R"], (rk, 128))
    Lv, Rv = shp(fv["L"], (P, rv)), shp(fv["R"], (rv, 128))
    Lk, Rk, Lv, Rv = _write_int4_cache(cache, dense["k"], dense["v"], Lk, Rk, Lv, Rv, T)
    qh = synth.queries(79, B, H * G, 128, 2.0)
    q = to_dev(qh)
    outs = [cache.decode(q, n_split=n).cpu().numpy() for n in (1, 5, 40, 0)]
    ref = _oracle(qh, T, dense["k"], dense["v"], Lk, Rk, Lv, Rv, 1, 4, G)
    for o in outs:
        assert rel_l2(o, ref).max() <= TOL, rel_l2(o, ref).max()
    for o in outs[1:]:
        assert rel_l2(o, outs[0]).max() <= 2 * 2.0 ** -11


@pytest.mark.parametrize("n_split", [0, 16])
def test_hybrid_int4_workload_sampled(n_split):
    """The int4 hybrid decode at the workload's full size (8 sequences x 8 KV heads x
    32K tokens, P=32, 1 sink, 4 window, rank 12), in the launch configuration the
    benchmark times (32 pages per wave), and with 16 chunks (64 pages per wave):
    random int4 factor codes in [-7, 7] and fp16 scales, dense pages from a seeded
    generator; sampled (sequence, KV head) pairs against the oracle."""
    R = _R()
    B, H, G, T, rk = 8, 8, 4, 32768, 12
    say(f"hybrid int4 workload sampled: B={B} H={H} T={T} n_split={n_split}")
    dev = torch.device("cuda")
    cache = R.PagedCache(B, H, G, 128, P, 1, 4, rk, rk, max_pages=T // P + 8, factor_fmt=R.FMT_INT4_G32)
    g = torch.Generator(device=dev)
    g.manual_seed(80)
    npg = T // P
    expect = opaged.page_table(T, P, 1, 4)
    cache.page_table[:, :, :npg] = torch.from_numpy(expect).to(dev)
    cache.lens.fill_(T)
    cache.host_lens[:] = T
    for n in ("lk", "rk", "lv", "rv"):
        a = getattr(cache, n)
        c = torch.randint(-7, 8, a.shape[:-1] + (2 * a.shape[-1],), generator=g, device=dev, dtype=torch.int16)
        a.copy_(((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).to(torch.uint8))
        # L entries ~ 0.1, R entries ~ 1 (scores of a few units)
        base = 0.1 / 7 if n in ("lk", "lv") else 1.0 / 7
        s = getattr(cache, n + "_s")
        s.copy_((base * (0.5 + torch.rand(s.shape, generator=g, device=dev))).half())
    cache.dense_k.copy_(torch.randn(cache.dense_k.shape, generator=g, device=dev).half())
    cache.dense_v.copy_(torch.randn(cache.dense_v.shape, generator=g, device=dev).half())
    q = torch.randn((B, H * G, 128), generator=g, device=dev)
    got = cache.decode(q, n_split=n_split).cpu().numpy()
    qn = q.cpu().numpy().astype(np.float64)
    for (b, h) in ((0, 0), (5, 3), (7, 7)):
        dec = {}
        for n, layout in (("lk", "key_L"), ("rk", "key_R"), ("lv", "value_L"), ("rv", "value_R")):
            dec[n] = _from_stored(getattr(cache, n)[b, h, :npg].cpu().numpy(),
                                  getattr(cache, n + "_s")[b, h, :npg].cpu().numpy(), layout, rk)[0][None, None]
        dk = np.zeros((1, 1, T, 128))
        dv = np.zeros((1, 1, T, 128))
        dks = cache.dense_k[b, h].cpu().numpy().astype(np.float64)
        dvs = np.swapaxes(cache.dense_v[b, h].cpu().numpy().astype(np.float64), -1, -2)
        for p in np.nonzero(expect < 0)[0]:
            slot = -1 - expect[p]
            dk[0, 0, p * P:(p + 1) * P] = dks[slot]
            dv[0, 0, p * P:(p + 1) * P] = dvs[slot]
        ref = _oracle(qn[b:b + 1, h * G:(h + 1) * G], T, dk, dv, dec["lk"], dec["rk"], dec["lv"], dec["rv"],
                      1, 4, G)
        err = rel_l2(got[b, h * G:(h + 1) * G], ref[0]).max()
        assert err <= TOL, ((b, h), err)
