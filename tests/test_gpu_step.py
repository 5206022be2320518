"""lrkv_decode_step (append, then decode, in one call) through the C ABI: bit for
bit the same outputs, cache contents and lengths as lrkv_append_latent followed by
lrkv_decode_attn, step after step, in every latent mode and format (fused into
three launches for the RoPE mode with fp16 latents, the append and the decode in
turn otherwise); one fused step against the float64 oracle; a rejected step
leaves everything unchanged."""
import numpy as np
import pytest
import torch

import synth
from oracle import attn as oattn
from tests.gpu_util import rel_l2, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as R
    R.load_library()


def _R():
    import rank_compressed_kv_amd as R
    return R


# name -> (B, U, s, g_q, d_h, r, theta, tau, fmt, mode, kernel the RoPE path takes)
CASES = {
    "glrd_r256_fw": (1, 8, 4, 1, 128, 256, 1e4, 96.0, "fp16", "rope"),
    "glrd_r64_generic": (2, 2, 2, 1, 64, 64, 1e4, 24.0, "fp16", "rope"),
    "gqa_r64_fp16": (2, 2, 1, 4, 128, 64, 5e5, 32.0, "fp16", "rope"),
    "gqa_r64_int4": (1, 2, 1, 4, 128, 64, 5e5, 32.0, "int4", "rope"),
    "absorbed_r128": (2, 2, 2, 1, 64, 128, 0.0, 48.0, "fp16", "absorbed"),
    "absorbed_r64_int4": (2, 2, 2, 1, 64, 64, 0.0, 24.0, "int4", "absorbed"),
}


def _pair(name, T, cap, seed):
    """Two caches with identical contents, the layer's B^k and the queries."""
    R = _R()
    B, U, s, gq, dh, r, th, tau, fmt, mode = CASES[name]
    f = R.FMT_FP16 if fmt == "fp16" else R.FMT_INT4_G32
    lay = synth.latent_layer(seed, B, U, T, r, s * dh, tau)
    caches = []
    for _ in range(2):
        c = R.LatentCache(B, U, s, gq, dh, r, cap, f, th)
        c.append(to_dev(lay["hk"]), to_dev(lay["hv"]))
        caches.append(c)
    return caches, lay["Bk"]


def _snapshot(c):
    parts = [c.hk, c.hv, c.lens] + [t for t in (c.sk, c.sv) if t is not None]
    return [t.clone() for t in parts]


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("n_new", [1, 3])
def test_step_equals_append_then_decode(name, n_new):
    R = _R()
    B, U, s, gq, dh, r, th, tau, fmt, mode = CASES[name]
    T0 = 32 * 40 - 2              # the steps cross a 32-token tile boundary
    say(f"decode_step vs append+decode: {name} n_new={n_new} T0={T0}")
    (ca, cb), Bk = _pair(name, T0, 32 * 48, 11)
    md = R.MODE_ROPE_RECON if mode == "rope" else R.MODE_ABSORBED
    bk = to_dev(Bk) if mode == "rope" else None
    qdim = dh if mode == "rope" else r
    for step in range(3):
        nk = to_dev(synth.latent_layer(100 + step, B, U, n_new, r, s * dh, tau)["hk"])
        nv = to_dev(synth.latent_layer(200 + step, B, U, n_new, r, s * dh, tau)["hv"])
        q = to_dev(synth.queries(300 + step, B, U * s * gq, qdim))
        oa = ca.step(md, nk, nv, q, bk)
        cb.append(nk, nv)
        ob = cb.decode(md, q, bk)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (name, step)
        for x, y in zip(_snapshot(ca), _snapshot(cb)):
            assert torch.equal(x, y), (name, step)
        assert ca.max_len == cb.max_len == T0 + n_new * (step + 1)
        assert int(ca.lens.max()) == ca.max_len


def test_step_explicit_query_positions():
    """q_pos given: the fused step rotates the query there, as append + decode does."""
    R = _R()
    B, U, s, gq, dh, r, th, tau, fmt, mode = CASES["glrd_r64_generic"]
    say("decode_step with explicit q_pos")
    (ca, cb), Bk = _pair("glrd_r64_generic", 700, 32 * 24, 13)
    nk = to_dev(synth.latent_layer(101, B, U, 1, r, s * dh, tau)["hk"])
    nv = to_dev(synth.latent_layer(102, B, U, 1, r, s * dh, tau)["hv"])
    q = to_dev(synth.queries(103, B, U * s * gq, dh))
    qp = to_dev(np.array([650, 699], np.int32))
    oa = ca.step(R.MODE_ROPE_RECON, nk, nv, q, to_dev(Bk), q_pos=qp)
    cb.append(nk, nv)
    ob = cb.decode(R.MODE_ROPE_RECON, q, to_dev(Bk), q_pos=qp)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)


def test_fused_step_against_oracle():
    """Config-2 geometry (the fused three-launch path): the output of a step that
    appends 2 tokens equals the float64 oracle on all the stored latents."""
    R = _R()
    B, U, s, gq, dh, r, th, tau, fmt, mode = CASES["glrd_r256_fw"]
    T0 = 32 * 64 + 5
    say(f"fused decode_step vs oracle: T0={T0}")
    lay = synth.latent_layer(17, B, U, T0 + 2, r, s * dh, tau)
    c = R.LatentCache(B, U, s, gq, dh, r, 32 * 72, R.FMT_FP16, th)
    c.append(to_dev(lay["hk"][:, :, :T0]), to_dev(lay["hv"][:, :, :T0]))
    q = synth.queries(18, B, U * s * gq, dh)
    out = c.step(R.MODE_ROPE_RECON, to_dev(lay["hk"][:, :, T0:]), to_dev(lay["hv"][:, :, T0:]), to_dev(q),
                 to_dev(lay["Bk"]))
    torch.cuda.synchronize()
    lens = np.full(B, T0 + 2, np.int64)
    ref = oattn.palu_decode(oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"]),
                            lay["Bk"].astype(np.float64), q, lens, s, gq, dh, th)
    err = rel_l2(out.cpu().numpy(), ref).max()
    assert err <= TOL, err
    assert int(c.lens[0]) == T0 + 2


@pytest.mark.parametrize("name", ["glrd_r256_fw", "gqa_r64_int4"])
def test_rejected_step_leaves_cache_unchanged(name):
    """Capacity exceeded by the append, and a workspace sized for the length before
    the append: both rejected before anything is enqueued."""
    R = _R()
    B, U, s, gq, dh, r, th, tau, fmt, mode = CASES[name]
    say(f"rejected decode_step: {name}")
    cap = 32 * 8
    (c, _), Bk = _pair(name, cap - 1, cap, 21)
    nk = to_dev(synth.latent_layer(22, B, U, 2, r, s * dh, tau)["hk"])
    nv = to_dev(synth.latent_layer(23, B, U, 2, r, s * dh, tau)["hv"])
    q = to_dev(synth.queries(24, B, U * s * gq, dh))
    out = torch.full((B, U * s * gq, r), 7.0, device="cuda")
    before = _snapshot(c)
    ws = c.workspace(R.MODE_ROPE_RECON)
    with pytest.raises(R.LrkvError) as e:
        R.decode_step(R.MODE_ROPE_RECON, c.desc, nk, nv, 2, q, to_dev(Bk), None, 0.0, out, ws, c.max_len)
    assert e.value.status == R._lib.LRKV_ERR_CAPACITY
    # one token fits, but the workspace only covers the length before the append
    need = R.decode_workspace_bytes(R.MODE_ROPE_RECON, c.desc, c.max_len + 1, 1)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(R.LrkvError) as e:
        R.decode_step(R.MODE_ROPE_RECON, c.desc, nk[:, :, :1].contiguous(), nv[:, :, :1].contiguous(), 1, q,
                      to_dev(Bk), None, 0.0, out, small, c.max_len, 1)
    assert e.value.status == R._lib.LRKV_ERR_WORKSPACE
    torch.cuda.synchronize()
    for x, y in zip(before, _snapshot(c)):
        assert torch.equal(x, y)
    assert bool((out == 7.0).all())


@pytest.mark.parametrize("fmt", ["fp16", "int4"])
def test_paged_step_equals_append_then_decode(fmt):
    """Hybrid paged cache: 40 steps across page boundaries (the page leaving the
    window is factored first in both), outputs, factors, dense pages, page table and
    lengths bit-identical to append + decode."""
    R = _R()
    B, H, G, P = 2, 2, 4, 32
    T0 = 32 * 9 + 20
    say(f"paged decode_step vs append+decode: {fmt}, T0={T0}, 40 steps")
    ff = R.FMT_FP16 if fmt == "fp16" else R.FMT_INT4_G32
    dense = synth.paged_dense(71, B, H, T0 + 40, 128)
    k = torch.from_numpy(dense["k"]).half().cuda()
    v = torch.from_numpy(dense["v"]).half().cuda()
    caches = []
    for _ in range(2):
        c = R.PagedCache(B, H, G, 128, P, 1, 4, 12, 12, max_pages=(T0 + 40) // P + 4, factor_fmt=ff)
        c.prefill(k[:, :, :T0].contiguous(), v[:, :, :T0].contiguous())
        caches.append(c)
    ca, cb = caches
    for i in range(40):
        t = T0 + i
        kt, vt = k[:, :, t:t + 1].contiguous(), v[:, :, t:t + 1].contiguous()
        q = to_dev(synth.queries(400 + i, B, H * G, 128))
        oa = ca.step(kt, vt, q)
        cb.append(kt, vt)
        ob = cb.decode(q)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), i
    for name in ("dense_k", "dense_v", "lk", "rk", "lv", "rv", "lk_s", "rk_s", "lv_s", "rv_s", "page_table",
                 "lens"):
        if getattr(ca, name) is not None:
            assert torch.equal(getattr(ca, name), getattr(cb, name)), name
