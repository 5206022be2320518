"""lrkv_decode_attn_noalloc against lrkv_decode_attn, through the C ABI: the same
kernels on the library's static scratch instead of a caller workspace. Two calls
in a row per case, the second on a smaller input (the scratch then still holds
the first call's data); each output must equal lrkv_decode_attn's bit for bit."""
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


def _both(mode, cache, q, bk, T, n_split=0):
    """(lrkv_decode_attn output, lrkv_decode_attn_noalloc output) at host length T."""
    import rank_compressed_kv_amd as R
    shape = (cache.B, cache.Hq if hasattr(cache, "Hq") else cache.H * cache.G,
             cache.d if mode == R.MODE_HYBRID_PAGED else cache.r)
    ws = torch.empty(R.decode_workspace_bytes(mode, cache.desc, T, n_split), dtype=torch.uint8, device="cuda")
    ref = torch.full(shape, np.nan, dtype=torch.float32, device="cuda")
    got = torch.full(shape, np.nan, dtype=torch.float32, device="cuda")
    R.decode_attn(mode, cache.desc, q, bk, None, 0.0, ref, ws, T, n_split)
    R.decode_attn_noalloc(mode, cache.desc, q, bk, None, 0.0, got, T, n_split)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def _set_len(cache, T):
    cache.lens.fill_(T)
    cache.host_lens[:] = T


@pytest.mark.parametrize("case", ["rope_fp16_glrd", "rope_int4_gqa", "absorbed_fp16", "absorbed_int4"])
def test_noalloc_latent_matches_decode_attn(case):
    import rank_compressed_kv_amd as R
    shapes = {  # B, U, s, gq, dh, r, fmt, theta, T1, T2
        "rope_fp16_glrd": (1, 8, 4, 1, 128, 256, R.FMT_FP16, 1e4, 8192, 1000),
        "rope_int4_gqa": (4, 8, 1, 4, 128, 64, R.FMT_INT4_G32, 5e5, 6000, 777),
        "absorbed_fp16": (4, 8, 4, 1, 128, 256, R.FMT_FP16, 0.0, 4096, 515),
        "absorbed_int4": (4, 8, 4, 1, 128, 256, R.FMT_INT4_G32, 0.0, 4096, 61),
    }
    B, U, s, gq, dh, r, fmt, theta, T1, T2 = shapes[case]
    mode = R.MODE_ABSORBED if theta == 0.0 else R.MODE_ROPE_RECON
    say(f"no-alloc decode: {case} T={T1} then T={T2}")
    lay = synth.latent_layer(91, B, U, T1, r, s * dh, 64.0)
    cache = R.LatentCache(B, U, s, gq, dh, r, -(-T1 // 32) * 32, fmt, theta)
    cache.append(to_dev(lay["hk"]), to_dev(lay["hv"]))
    qdim = r if mode == R.MODE_ABSORBED else dh
    q = to_dev(synth.queries(92, B, U * s * gq, qdim, 2.0))
    bk = None if mode == R.MODE_ABSORBED else to_dev(lay["Bk"])
    for T in (T1, T2):
        _set_len(cache, T)
        ref, got = _both(mode, cache, q, bk, T)
        assert np.isfinite(ref).all()
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), (case, T)


@pytest.mark.parametrize("factor_fmt_name", ["fp16", "int4"])
def test_noalloc_hybrid_matches_decode_attn(factor_fmt_name):
    import rank_compressed_kv_amd as R
    fmt = R.FMT_FP16 if factor_fmt_name == "fp16" else R.FMT_INT4_G32
    B, H, G, T1, T2 = 4, 8, 4, 32 * 300 + 7, 32 * 40 + 3
    say(f"no-alloc decode: hybrid {factor_fmt_name} factors T={T1} then T={T2}")
    dense = synth.paged_dense(93, B, H, T1, 128)
    q = to_dev(synth.queries(94, B, H * G, 128, 2.0))
    for T in (T1, T2):
        cache = R.PagedCache(B, H, G, 128, 32, 1, 4, 12, 12, max_pages=(T + 31) // 32 + 1, factor_fmt=fmt)
        cache.prefill(to_dev(np.ascontiguousarray(dense["k"][:, :, :T])),
                      to_dev(np.ascontiguousarray(dense["v"][:, :, :T])))
        ref, got = _both(R.MODE_HYBRID_PAGED, cache, q, None, T)
        assert np.isfinite(ref).all()
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), (factor_fmt_name, T)


def test_noalloc_rejects_beyond_scratch():
    """A call needing more than the static scratch is refused before anything is
    enqueued (the output keeps its bytes); a following call within the limit works."""
    import rank_compressed_kv_amd as R
    from rank_compressed_kv_amd import _lib as L
    B, U, s, dh, r, T = 4, 8, 4, 128, 256, 32768
    say(f"no-alloc decode: beyond the scratch, B={B} T={T} n_split=1024")
    cache = R.LatentCache(B, U, s, 1, dh, r, T, R.FMT_FP16, 0.0)
    _set_len(cache, T)
    q = to_dev(synth.queries(95, B, U * s, r))
    assert R.decode_workspace_bytes(R.MODE_ABSORBED, cache.desc, T, 1024) > L.NOALLOC_SCRATCH_BYTES
    out = torch.full((B, U * s, r), 1.5, dtype=torch.float32, device="cuda")
    with pytest.raises(R.LrkvError) as ei:
        R.decode_attn_noalloc(R.MODE_ABSORBED, cache.desc, q, None, None, 0.0, out, T, 1024)
    assert ei.value.status == L.LRKV_ERR_SCRATCH
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == 1.5).all()
    R.decode_attn_noalloc(R.MODE_ABSORBED, cache.desc, q, None, None, 0.0, out, T, 0)
    torch.cuda.synchronize()
    assert np.isfinite(out.cpu().numpy()).all()
