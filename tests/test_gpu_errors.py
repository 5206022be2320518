"""A rejected call leaves device state unchanged: after an append or decode that
the library refuses (capacity, workspace, bad arguments), every cache buffer, the
device lengths and the output buffer hold exactly the bytes they held before."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as R
    R.load_library()


def _snap(tensors):
    torch.cuda.synchronize()
    return [t.clone() for t in tensors]


def _same(before, after):
    torch.cuda.synchronize()
    for a, b in zip(before, after):
        assert torch.equal(a.view(torch.uint8) if a.dtype != torch.uint8 else a,
                           b.view(torch.uint8) if b.dtype != torch.uint8 else b)


def _expect(status, fn):
    import rank_compressed_kv_amd as R
    with pytest.raises(R.LrkvError) as ei:
        fn()
    assert ei.value.status == status, (ei.value.status, status)


@pytest.mark.parametrize("fmt_name", ["fp16", "int4"])
def test_rejected_latent_calls_leave_cache_unchanged(fmt_name):
    import rank_compressed_kv_amd as R
    from rank_compressed_kv_amd import _lib as L
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"rejected latent calls: {fmt_name}")
    B, U, s, dh, r, cap, T = 2, 2, 2, 64, 64, 128, 100
    lay = synth.latent_layer(41, B, U, T, r, s * dh, 24.0)
    cache = R.LatentCache(B, U, s, 1, dh, r, cap, fmt, 1e4)
    cache.append(to_dev(lay["hk"]), to_dev(lay["hv"]))
    bufs = [t for t in (cache.hk, cache.hv, cache.sk, cache.sv, cache.lens) if t is not None]
    q = to_dev(synth.queries(42, B, U * s, dh))
    bk = to_dev(lay["Bk"])
    out = torch.full((B, U * s, r), 7.25, dtype=torch.float32, device="cuda")
    before = _snap(bufs + [out])
    # capacity: 100 + 29 > 128
    nk = to_dev(np.ones((B, U, 29, r), np.float32))
    _expect(L.LRKV_ERR_CAPACITY, lambda: R.append_latent(R.MODE_ROPE_RECON, cache.desc, nk, nk, 29, T))
    # workspace one byte short, and missing
    need = R.decode_workspace_bytes(R.MODE_ROPE_RECON, cache.desc, T)
    ws_small = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    _expect(L.LRKV_ERR_WORKSPACE, lambda: R.decode_attn(R.MODE_ROPE_RECON, cache.desc, q, bk, None, 0.0, out,
                                                        ws_small, T))
    _expect(L.LRKV_ERR_WORKSPACE, lambda: R.decode_attn(R.MODE_ROPE_RECON, cache.desc, q, bk, None, 0.0, out,
                                                        None, T))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    # length bound past the capacity; B^k missing on the RoPE path; B^k given on the absorbed path
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.decode_attn(R.MODE_ROPE_RECON, cache.desc, q, bk, None, 0.0, out,
                                                          ws, cap + 1))
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.decode_attn(R.MODE_ROPE_RECON, cache.desc, q, None, None, 0.0, out,
                                                          ws, T))
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.decode_attn(R.MODE_ABSORBED, cache.desc, q, bk, None, 0.0, out,
                                                          ws, T))
    # a descriptor with an unsupported rank that still points at this cache's buffers
    bad = L.LatentCacheDesc.from_buffer_copy(cache.desc)
    bad.rank = 36
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.append_latent(R.MODE_ROPE_RECON, bad, nk, nk, 1, T))
    _same(before, bufs + [out])
    # the same cache still accepts a valid call afterwards
    R.decode_attn(R.MODE_ROPE_RECON, cache.desc, q, bk, None, 0.0, out, ws, T)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()


def test_rejected_paged_calls_leave_cache_unchanged():
    import rank_compressed_kv_amd as R
    from rank_compressed_kv_amd import _lib as L
    say("rejected paged calls")
    B, H, G, T, max_pages = 2, 2, 4, 32 * 7 + 5, 8
    cache = R.PagedCache(B, H, G, 128, 32, 1, 4, 12, 12, max_pages=max_pages)
    dense = synth.paged_dense(43, B, H, T, 128)
    cache.prefill(to_dev(dense["k"]), to_dev(dense["v"]))
    bufs = [cache.dense_k, cache.dense_v, cache.lk, cache.rk, cache.lv, cache.rv, cache.page_table, cache.lens]
    q = to_dev(synth.queries(44, B, H * G, 128))
    out = torch.full((B, H * G, 128), -3.5, dtype=torch.float32, device="cuda")
    before = _snap(bufs + [out])
    # capacity: 229 + 28 > 256
    nk = torch.zeros((B, H, 28, 128), dtype=torch.float16, device="cuda")
    _expect(L.LRKV_ERR_CAPACITY, lambda: R.append_latent(R.MODE_HYBRID_PAGED, cache.desc, nk, nk, 28, T))
    need = R.decode_workspace_bytes(R.MODE_HYBRID_PAGED, cache.desc, T)
    ws_small = torch.zeros(need - 4, dtype=torch.uint8, device="cuda")
    _expect(L.LRKV_ERR_WORKSPACE, lambda: R.decode_attn(R.MODE_HYBRID_PAGED, cache.desc, q, None, None, 0.0, out,
                                                        ws_small, T))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.decode_attn(R.MODE_HYBRID_PAGED, cache.desc, q, None, None, 0.0, out,
                                                          ws, max_pages * 32 + 1))
    # factorisation from a caller buffer shorter than a page, and an over-long sweep limit
    pages = torch.zeros((1, 3), dtype=torch.int32, device="cuda")
    src = torch.zeros((B, H, 31, 128), dtype=torch.float16, device="cuda")
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.factor_page(cache.desc, pages, 1, src, src, 31))
    _expect(L.LRKV_ERR_INVALID_ARG, lambda: R.factor_page(cache.desc, pages, 1, max_sweeps=101))
    # an unsupported page size in a descriptor that points at this cache's buffers
    bad = L.PagedCacheDesc.from_buffer_copy(cache.desc)
    bad.page_size = 16
    _expect(L.LRKV_ERR_UNSUPPORTED, lambda: R.append_latent(R.MODE_HYBRID_PAGED, bad, nk, nk, 1, T))
    _same(before, bufs + [out])
    R.decode_attn(R.MODE_HYBRID_PAGED, cache.desc, q, None, None, 0.0, out, ws, T)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
