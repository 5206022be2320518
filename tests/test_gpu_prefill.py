"""GPU parity of chunked-prefill attention (reconstruct-with-RoPE path, fp16
latents, rank 256, head_dim 128) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from oracle import attn as oattn
from tests.gpu_util import rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3
R, DH, THETA = 256, 128, 1e4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as Rk
    Rk.load_library()


def _setup(seed, B, U, s, gq, T_end, cap):
    """Cache filled to T_end tokens per sequence with config-2 style latents."""
    import rank_compressed_kv_amd as Rk
    lay = synth.latent_layer(seed, B, U, T_end, R, s * DH, 96.0)
    c = Rk.LatentCache(B, U, s, gq, DH, R, cap, Rk.FMT_FP16, THETA)
    c.append(to_dev(lay["hk"].astype(np.float32)), to_dev(lay["hv"].astype(np.float32)))
    bk16 = lay["Bk"].astype(np.float16)
    return c, lay, bk16


@pytest.mark.parametrize("B,U,s,gq,T0,M,cap", [(2, 2, 4, 1, 300, 100, 512), (1, 2, 2, 2, 64, 40, 128),
                                                (2, 1, 4, 1, 0, 77, 96), (1, 1, 2, 2, 1000, 1, 1024),
                                                (1, 1, 4, 1, 31, 129, 192), (1, 2, 2, 4, 500, 70, 640),
                                                (1, 1, 2, 4, 3000, 200, 3264)])
def test_prefill_parity(B, U, s, gq, T0, M, cap):
    """A chunk of M tokens appended after T0 cached ones (all sequences at the same
    length), causal attention of every chunk query against the oracle on the stored
    fp16 latents."""
    say(f"prefill parity: B={B} U={U} s={s} gq={gq} T0={T0} M={M}")
    c, lay, bk16 = _setup(41, B, U, s, gq, T0 + M, cap)
    Hq = U * s * gq
    q = synth.queries(42, B * M, Hq, DH, 1.0).reshape(B, M, Hq, DH)
    p0 = np.full(B, T0, np.int32)
    got = c.prefill_attn(to_dev(q), to_dev(bk16), to_dev(p0)).cpu().numpy()
    ref = oattn.palu_prefill(oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"]),
                             bk16.astype(np.float64), q, p0, s, gq, DH, THETA)
    err = rel_l2(got.reshape(B * M, Hq, R), ref.reshape(B * M, Hq, R))
    say(f"  max rel-L2 {err.max():.3e} (tolerance {TOL})")
    assert err.max() <= TOL, err.max()


def test_prefill_ragged_positions():
    """Sequences whose chunks start at different positions: every sequence holds
    latents to the longest length, and lens[b] = p0[b] + M marks its own end (rows
    past it must not be read)."""
    import rank_compressed_kv_amd as Rk
    B, U, s, gq, M, cap = 3, 1, 4, 1, 50, 512
    T0 = [10, 333, 200]
    say(f"prefill ragged: p0={T0} M={M}")
    lay = synth.latent_layer(43, B, U, max(T0) + M, R, s * DH, 96.0)
    c = Rk.LatentCache(B, U, s, gq, DH, R, cap, Rk.FMT_FP16, THETA)
    c.append(to_dev(lay["hk"].astype(np.float32)), to_dev(lay["hv"].astype(np.float32)))
    lens = (np.array(T0) + M).astype(np.int32)
    c.lens.copy_(torch.from_numpy(lens))
    c.host_lens[:] = lens
    bk16 = lay["Bk"].astype(np.float16)
    Hq = U * s * gq
    q = synth.queries(44, B * M, Hq, DH, 1.5).reshape(B, M, Hq, DH)
    p0 = np.array(T0, np.int32)
    got = c.prefill_attn(to_dev(q), to_dev(bk16), to_dev(p0)).cpu().numpy()
    ref = oattn.palu_prefill(oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"]),
                             bk16.astype(np.float64), q, p0, s, gq, DH, THETA)
    err = rel_l2(got.reshape(B * M, Hq, R), ref.reshape(B * M, Hq, R))
    say(f"  max rel-L2 {err.max():.3e} (tolerance {TOL})")
    assert err.max() <= TOL, err.max()


def test_prefill_full_size_sampled():
    """Llama-2-7B layer (8 units x 4 heads, r 256): a 512-token chunk at the end of a
    65536-token context, the configuration the benchmark times. Latents from a seeded
    generator on the GPU (config-2 spectrum); sampled (token, head) rows against the
    oracle's decode at each row's length (the prefill rows' definition)."""
    import rank_compressed_kv_amd as Rk
    B, U, s, gq, T, M, CH = 1, 8, 4, 1, 65536, 512, 16384
    say(f"prefill full size: T={T} M={M}")
    dev = torch.device("cuda")
    bk16 = synth.latent_layer(45, 1, U, 32, R, s * DH, 96.0)["Bk"].astype(np.float16)
    c = Rk.LatentCache(B, U, s, gq, DH, R, T, Rk.FMT_FP16, THETA)
    g = torch.Generator(device=dev)
    g.manual_seed(45)
    sq = torch.exp(-torch.arange(R, device=dev, dtype=torch.float32) / (2 * 96.0))
    samples = ((0, 0), (255, 13), (511, 31))
    units = sorted({j // s for _, j in samples})
    keep_k = {u: [] for u in units}
    keep_v = {u: [] for u in units}
    for _ in range(0, T, CH):
        hk = torch.randn((B, U, CH, R), generator=g, device=dev) * sq
        hv = torch.randn((B, U, CH, R), generator=g, device=dev) * sq
        c.append(hk, hv)
        for u in units:
            keep_k[u].append(hk[0, u].cpu().numpy())
            keep_v[u].append(hv[0, u].cpu().numpy())
    Hq = U * s * gq
    q = synth.queries(46, M, Hq, DH, 1.0).reshape(B, M, Hq, DH)
    p0 = np.array([T - M], np.int32)
    got = c.prefill_attn(to_dev(q), to_dev(bk16), to_dev(p0)).cpu().numpy()
    for (m, j) in samples:
        n = T - M + m + 1
        u = j // (s * gq)
        hk = oattn.stored_fp16(np.concatenate(keep_k[u])[None, None, :n])
        hv = oattn.stored_fp16(np.concatenate(keep_v[u])[None, None, :n])
        ref = oattn.palu_decode(hk, hv, bk16[u:u + 1].astype(np.float64), q[:, m, u * s * gq:(u + 1) * s * gq],
                                [n], s, gq, DH, THETA)
        err = rel_l2(got[0, m, j], ref[0, j - u * s * gq])
        say(f"  row {m} head {j}: rel-L2 {err:.3e} (tolerance {TOL})")
        assert err <= TOL, (m, j)


def test_prefill_without_rope():
    """rope_theta = 0: plain reconstruct-and-attend (no rotation on either side)."""
    import rank_compressed_kv_amd as Rk
    B, U, s, gq, T0, M, cap = 1, 1, 4, 1, 200, 60, 288
    say(f"prefill no RoPE: T0={T0} M={M}")
    lay = synth.latent_layer(47, B, U, T0 + M, R, s * DH, 96.0)
    c = Rk.LatentCache(B, U, s, gq, DH, R, cap, Rk.FMT_FP16, 0.0)
    c.append(to_dev(lay["hk"].astype(np.float32)), to_dev(lay["hv"].astype(np.float32)))
    bk16 = lay["Bk"].astype(np.float16)
    Hq = U * s * gq
    q = synth.queries(48, B * M, Hq, DH, 1.0).reshape(B, M, Hq, DH)
    p0 = np.full(B, T0, np.int32)
    got = c.prefill_attn(to_dev(q), to_dev(bk16), to_dev(p0)).cpu().numpy()
    ref = oattn.palu_prefill(oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"]),
                             bk16.astype(np.float64), q, p0, s, gq, DH, 0.0)
    err = rel_l2(got.reshape(B * M, Hq, R), ref.reshape(B * M, Hq, R))
    say(f"  max rel-L2 {err.max():.3e} (tolerance {TOL})")
    assert err.max() <= TOL, err.max()
