"""GPU parity of the Palu latent-cache path (append, RoPE reconstruction, absorbed
query, split merge) against the float64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import synth
from oracle import attn as oattn
from oracle import codec as ocodec
from tests.gpu_util import (hk_int4_codes, hv_fp16_tokens, hv_int4_codes, rel_l2, say, sv_tokens,
                            to_dev)

pytestmark = pytest.mark.gpu

TOL = 2e-3      # rel-L2 per (sequence, head) on attention outputs


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as R
    R.load_library()


def _R():
    import rank_compressed_kv_amd as R
    return R


# shapes: name -> (B, U, s, g_q, d_h, r, theta, tau)
SHAPES = {
    "tiny_glrd": (1, 2, 2, 1, 64, 32, 1e4, 24.0),
    "llama2_glrd": (1, 8, 4, 1, 128, 256, 1e4, 96.0),
    "llama3_gqa": (2, 8, 1, 4, 128, 64, 5e5, 32.0),
    "llama3_gqa_r32": (2, 8, 1, 4, 128, 32, 5e5, 32.0),
}


def _make(name, T, cap, fmt, seed, q_scale=1.0, ragged=(), theta=None, mixed=False):
    R = _R()
    B, U, s, gq, dh, r, th, tau = SHAPES[name]
    th = th if theta is None else theta
    lay = synth.latent_layer(seed, B, U, T, r, s * dh, tau)
    hk, hv, Bk = lay["hk"], lay["hv"], lay["Bk"]
    if mixed:
        hk, Bk = synth.hadamard_mixed(hk, Bk)
        hv, _ = synth.hadamard_mixed(hv, lay["Bv"])
    q = synth.queries(seed + 1000, B, U * s * gq, dh, q_scale)
    cache = R.LatentCache(B, U, s, gq, dh, r, cap, fmt, th)
    cache.append(to_dev(hk), to_dev(hv))
    lens = np.full(B, T, np.int64)
    for b, cut in enumerate(ragged[:B]):
        lens[b] = T - cut
    if len(ragged):
        cache.lens.copy_(torch.from_numpy(lens.astype(np.int32)))
        cache.host_lens[:] = lens
    store = oattn.stored_fp16 if fmt == R.FMT_FP16 else oattn.stored_int4
    return dict(cache=cache, hk=hk, hv=hv, Bk=Bk, q=q, lens=lens, s=s, gq=gq, dh=dh, r=r, theta=th,
                sk=store(hk), sv=store(hv))


def _oracle_rope(c, q_pos=None):
    return oattn.palu_decode(c["sk"], c["sv"], c["Bk"].astype(np.float64), c["q"], c["lens"], c["s"],
                             c["gq"], c["dh"], c["theta"], q_pos=q_pos)


def _gpu_rope(c, n_split=0, q_pos=None):
    R = _R()
    qp = None if q_pos is None else to_dev(np.asarray(q_pos, np.int32))
    out = c["cache"].decode(R.MODE_ROPE_RECON, to_dev(c["q"]), to_dev(c["Bk"]), qp, n_split=n_split)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# ----------------------------------------------------------------------------- append

def test_append_fp16_bitexact():
    R = _R()
    say("append fp16: B=2 U=3 r=64, appends of 37, 1, 26 tokens")
    rng = np.random.default_rng(11)
    cache = R.LatentCache(2, 3, 1, 1, 64, 64, 128, R.FMT_FP16, 0.0)
    chunks = []
    for n in (37, 1, 26):
        a = (rng.standard_normal((2, 3, n, 64)) * 3).astype(np.float32)
        a[0, 0, 0, :4] = [65519.0, 65520.0, 1e-8, -2.0 ** -25]     # overflow / subnormal edges
        v = (rng.standard_normal((2, 3, n, 64))).astype(np.float32)
        cache.append(to_dev(a), to_dev(v))
        chunks.append((a, v))
    torch.cuda.synchronize()
    k_all = np.concatenate([c[0] for c in chunks], axis=2)
    v_all = np.concatenate([c[1] for c in chunks], axis=2)
    with np.errstate(over="ignore"):
        ek, ev = k_all.astype(np.float16), v_all.astype(np.float16)
    got_k = cache.hk.cpu().numpy()[:, :, :64]
    got_v = hv_fp16_tokens(cache.hv)[:, :, :64]
    assert np.array_equal(got_k.view(np.uint16), ek.view(np.uint16))
    assert np.array_equal(got_v.view(np.uint16), ev.view(np.uint16))
    assert cache.lens.cpu().tolist() == [64, 64]


def test_append_int4_bitexact():
    R = _R()
    say("append int4: B=2 U=2 r=64, appends of 5, 1, 26, 1 tokens (odd offsets)")
    rng = np.random.default_rng(12)
    cache = R.LatentCache(2, 2, 1, 4, 128, 64, 64, R.FMT_INT4_G32, 5e5)
    ks, vs = [], []
    for n in (5, 1, 26, 1):
        k = (rng.standard_normal((2, 2, n, 64)) * rng.uniform(0.01, 20)).astype(np.float32)
        v = (rng.standard_normal((2, 2, n, 64)) * rng.uniform(0.01, 20)).astype(np.float32)
        k[0, 0, 0, :32] = 0.0                                          # all-zero group
        k[0, 1, 0, :32] = 0.0
        k[0, 1, 0, 7] = -3.0                                           # single nonzero
        k[1, 0, 0, :32] = np.float32(1.0) * np.array([7.0] + [2.5, 3.5, -2.5, 0.5] * 7 + [1.5, 6.5, -6.5], np.float32)
        v[1, 1, 0, 32:] = np.array([7.0] + [(k + 0.5) for k in range(-4, 3)] * 4 + [0.5, 1.5, -0.5], np.float32)
        # exact ties of an inexact scale: amax 1 -> s16 = fp16(fp32(1) / 7), x = s16 (k + 1/2)
        s16 = np.float64(np.float16(np.float32(1.0) / np.float32(7.0)))
        ties = np.array([1.0] + [s16 * (j + 0.5) for j in (0, 1, 2, 3, -1, -4, -2, -3)] * 3
                        + [s16 * 4.5, -s16 * 5.5, s16 * 6.5, -s16 * 6.5, s16 * 5.5, -s16 * 0.5, s16 * 1.5],
                        np.float32)
        k[1, 1, 0, 32:] = ties
        v[0, 0, 0, :32] = -ties
        cache.append(to_dev(k), to_dev(v))
        ks.append(k)
        vs.append(v)
    torch.cuda.synchronize()
    K = np.concatenate(ks, axis=2)
    V = np.concatenate(vs, axis=2)
    T = K.shape[2]
    ck, sk = ocodec.quantize(K)
    cv, sv = ocodec.quantize(V)
    assert np.array_equal(hk_int4_codes(cache.hk)[:, :, :T], ck)
    assert np.array_equal(cache.sk.cpu().numpy()[:, :, :T].view(np.uint16), sk.view(np.uint16))
    assert np.array_equal(hv_int4_codes(cache.hv)[:, :, :T], cv)
    assert np.array_equal(sv_tokens(cache.sv)[:, :, :T].view(np.uint16), sv.view(np.uint16))
    # packed bytes themselves: dims 2i / 2i+1 in the low / high nibble
    assert np.array_equal(cache.hk.cpu().numpy()[:, :, :T], ocodec.pack(ck))


# ----------------------------------------------------------------------------- RoPE path

@pytest.mark.parametrize("name,T,cap,ragged,q_scale", [
    ("tiny_glrd", 256, 256, (), 1.0),
    ("tiny_glrd", 200, 256, (), 6.0),
    ("llama2_glrd", 2048, 2048, (), 1.0),
    ("llama2_glrd", 1000, 1024, (), 8.0),
    ("llama3_gqa", 1111, 1152, (0, 333), 1.0),
])
def test_rope_fp16_parity(name, T, cap, ragged, q_scale):
    R = _R()
    say(f"rope fp16 parity: {name} T={T} ragged={ragged} q_scale={q_scale}")
    c = _make(name, T, cap, R.FMT_FP16, seed=21, q_scale=q_scale, ragged=ragged)
    got = _gpu_rope(c)
    ref = _oracle_rope(c)
    err = rel_l2(got, ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("name,T,cap,ragged", [
    ("llama3_gqa", 1500, 1536, (0, 77)),
    ("llama2_glrd", 700, 704, ()),
])
def test_rope_int4_parity(name, T, cap, ragged):
    R = _R()
    say(f"rope int4 parity: {name} T={T} ragged={ragged}")
    c = _make(name, T, cap, R.FMT_INT4_G32, seed=22, ragged=ragged, mixed=True)
    err = rel_l2(_gpu_rope(c), _oracle_rope(c))
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("fmt_name,T,cap,ragged,n_split", [
    ("int4", 31, 32, (), 0),                 # one partial tile
    ("int4", 4097, 4128, (0, 4000), 0),      # ragged: 97 tokens in sequence 1
    ("fp16", 777, 800, (0, 1), 3),
    ("int4", 2000, 2048, (5, 0), 1),         # one chunk of 63 tiles per (sequence, unit)
    ("fp16", 32, 32, (), 0),                 # exactly one tile
])
def test_rope_gqa_edges(fmt_name, T, cap, ragged, n_split):
    """Grouped-query units (one KV head, 4 query heads, rank 64): tile tails,
    ragged lengths and chunkings of the reconstruct-then-rotate kernel."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"rope gqa edges: {fmt_name} T={T} ragged={ragged} n_split={n_split}")
    c = _make("llama3_gqa", T, cap, fmt, seed=26, ragged=ragged, mixed=fmt_name == "int4")
    err = rel_l2(_gpu_rope(c, n_split=n_split), _oracle_rope(c))
    say(f"  max rel-L2 {err.max():.3g}")
    assert err.max() <= TOL, err.max()


def test_rope_gqa_split_independence():
    R = _R()
    say("rope gqa split independence: llama3_gqa int4 T=3000, n_split 1/2/5/auto")
    c = _make("llama3_gqa", 3000, 3008, R.FMT_INT4_G32, seed=27, mixed=True)
    ref = _oracle_rope(c)
    outs = [_gpu_rope(c, n_split=n) for n in (1, 2, 5, 0)]
    for o in outs:
        assert rel_l2(o, ref).max() <= TOL
        assert rel_l2(o, outs[0]).max() <= 2 * 2.0 ** -11


@pytest.mark.parametrize("fmt_name,n_split", [("int4", 0), ("int4", 3), ("fp16", 0)])
def test_rope_gqa_rank32(fmt_name, n_split):
    """Grouped-query units at rank 32 (one 32-element scale group per token)."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"rope gqa rank 32: {fmt_name} T=900 ragged=(0, 45) n_split={n_split}")
    c = _make("llama3_gqa_r32", 900, 928, fmt, seed=28, ragged=(0, 45), mixed=fmt_name == "int4")
    err = rel_l2(_gpu_rope(c, n_split=n_split), _oracle_rope(c))
    say(f"  max rel-L2 {err.max():.3g}")
    assert err.max() <= TOL, err.max()


def _poison_tail(cache, lens, int4):
    """Every cache entry at or past its sequence's length becomes NaN (fp16
    latents and scales) or 0xFF code bytes: memory the caller never wrote."""
    nan = float("nan")
    blk = 32
    for b, n in enumerate(int(x) for x in lens):
        nb, pos = n // blk, n % blk
        cache.hk[b, :, n:] = 255 if int4 else nan
        if int4:
            cache.sk[b, :, n:] = nan
            cache.hv[b, :, nb + 1:] = 255
            cache.sv[b, :, nb + 1:] = nan
            if nb < cache.sv.shape[2]:
                cache.hv[b, :, nb, :, (pos + 1) // 2:] = 255
                cache.sv[b, :, nb, :, pos:] = nan
        else:
            cache.hv[b, :, nb + 1:] = nan
            if nb < cache.hv.shape[2]:
                cache.hv[b, :, nb, :, pos:] = nan


@pytest.mark.parametrize("name,fmt_name,T,cap,ragged,n_split", [
    ("llama3_gqa", "int4", 1000, 1056, (0, 333), 0),
    ("llama3_gqa", "int4", 1000, 1056, (17, 333), 3),
    ("llama3_gqa", "int4", 31, 64, (), 0),
    ("llama3_gqa_r32", "int4", 700, 736, (0, 5), 0),
    ("llama3_gqa", "fp16", 1000, 1056, (0, 333), 0),
    ("llama2_glrd", "fp16", 1500, 1536, (), 0),
    ("llama2_glrd", "fp16", 1500, 1536, (), 5),
    ("llama2_glrd", "int4", 700, 736, (), 0),
    ("tiny_glrd", "fp16", 200, 256, (), 0),
    ("tiny_glrd", "int4", 201, 256, (), 0),
])
def test_rope_poisoned_tail(name, fmt_name, T, cap, ragged, n_split):
    """Cache entries past each sequence's end hold NaN: nothing of them may reach
    the result (several tiles can share one score accumulator, where a NaN key
    would spread to the other tiles' columns)."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"rope poisoned tail: {name} {fmt_name} T={T} ragged={ragged} n_split={n_split}")
    c = _make(name, T, cap, fmt, seed=29, ragged=ragged, mixed=fmt_name == "int4")
    _poison_tail(c["cache"], c["lens"], fmt_name == "int4")
    torch.cuda.synchronize()
    got = _gpu_rope(c, n_split=n_split)
    assert np.isfinite(got).all()
    err = rel_l2(got, _oracle_rope(c))
    say(f"  max rel-L2 {err.max():.3g}")
    assert err.max() <= TOL, err.max()


def test_rope_split_independence():
    R = _R()
    say("rope split independence: llama2_glrd T=1500, n_split 1/3/7/auto")
    c = _make("llama2_glrd", 1500, 1504, R.FMT_FP16, seed=23, q_scale=4.0)
    ref = _oracle_rope(c)
    outs = [_gpu_rope(c, n_split=n) for n in (1, 3, 7, 0)]
    # p enters the value MFMA as fp16 relative to each chunk's own maximum, so two
    # chunkings differ by at most two fp16 roundings of p (unit roundoff 2^-11)
    for o in outs:
        assert rel_l2(o, ref).max() <= TOL
        assert rel_l2(o, outs[0]).max() <= 2 * 2.0 ** -11


def test_rope_query_position():
    R = _R()
    say("rope explicit q_pos: tiny_glrd T=256")
    c = _make("tiny_glrd", 256, 256, R.FMT_FP16, seed=24)
    a = _gpu_rope(c, q_pos=[255])
    assert rel_l2(a, _gpu_rope(c)).max() <= 1e-6
    b = _gpu_rope(c, q_pos=[17])
    assert rel_l2(b, _oracle_rope(c, q_pos=[17])).max() <= TOL


def test_rope_off_equals_absorbed():
    """theta = 0: reconstruct path == absorbed path with q' = q (B^k)^T."""
    R = _R()
    say("rope theta=0 vs absorbed: llama2_glrd T=900")
    c = _make("llama2_glrd", 900, 928, R.FMT_FP16, seed=25, theta=0.0)
    got_r = _gpu_rope(c)
    B, U, s, dh = 1, 8, 4, 128
    Bk = c["Bk"].astype(np.float64)
    qa = np.stack([[c["q"][b, j] @ Bk[j // s][:, (j % s) * dh:(j % s + 1) * dh].T for j in range(32)]
                   for b in range(B)]).astype(np.float32)
    got_a = c["cache"].decode(R.MODE_ABSORBED, to_dev(qa), sm_scale=1 / np.sqrt(dh))
    torch.cuda.synchronize()
    got_a = got_a.cpu().numpy()
    ref = _oracle_rope(c)
    assert rel_l2(got_r, ref).max() <= TOL
    assert rel_l2(got_a, ref).max() <= TOL


# ----------------------------------------------------------------------------- absorbed path

@pytest.mark.parametrize("fmt_name,B,T,cap,r,s", [("fp16", 3, 700, 704, 256, 4), ("fp16", 2, 4096, 4096, 256, 4),
                                                  ("int4", 2, 999, 1024, 256, 4), ("int4", 3, 2000, 2048, 128, 4),
                                                  ("int4", 2, 515, 544, 64, 2), ("int4", 1, 77, 96, 32, 2),
                                                  ("fp16", 2, 333, 352, 64, 2)])
def test_absorbed_parity(fmt_name, B, T, cap, r, s):
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"absorbed parity: {fmt_name} B={B} T={T} r={r} heads/unit={s}")
    U, dh = 8, 128
    lay = synth.latent_layer(31, B, U, T, r, s * dh, 96.0)
    qa = synth.queries(32, B, U * s, r, 3.0)
    cache = R.LatentCache(B, U, s, 1, dh, r, cap, fmt, 0.0)
    cache.append(to_dev(lay["hk"]), to_dev(lay["hv"]))
    lens = np.array([T - 53 * b for b in range(B)])
    cache.lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    cache.host_lens[:] = lens
    got = cache.decode(R.MODE_ABSORBED, to_dev(qa))
    torch.cuda.synchronize()
    store = oattn.stored_fp16 if fmt == R.FMT_FP16 else oattn.stored_int4
    ref = oattn.palu_decode_absorbed(store(lay["hk"]), store(lay["hv"]), qa, lens, s, 1, dh)
    err = rel_l2(got.cpu().numpy(), ref)
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("fmt_name,B,T,cap,r,s", [("fp16", 3, 700, 736, 256, 4), ("int4", 2, 999, 1024, 256, 4),
                                                  ("int4", 2, 515, 544, 64, 2), ("fp16", 2, 333, 352, 64, 2)])
def test_absorbed_poisoned_tail(fmt_name, B, T, cap, r, s):
    """Absorbed path with NaN (fp16) or 0xFF codes and NaN scales (int4) in every
    cache entry past each sequence's end."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"absorbed poisoned tail: {fmt_name} B={B} T={T} r={r} heads/unit={s}")
    U, dh = 8, 128
    lay = synth.latent_layer(33, B, U, T, r, s * dh, 96.0)
    qa = synth.queries(34, B, U * s, r, 3.0)
    cache = R.LatentCache(B, U, s, 1, dh, r, cap, fmt, 0.0)
    cache.append(to_dev(lay["hk"]), to_dev(lay["hv"]))
    lens = np.array([T - 53 * b for b in range(B)])
    cache.lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    cache.host_lens[:] = lens
    _poison_tail(cache, lens, fmt_name == "int4")
    got = cache.decode(R.MODE_ABSORBED, to_dev(qa)).cpu().numpy()
    assert np.isfinite(got).all()
    store = oattn.stored_fp16 if fmt == R.FMT_FP16 else oattn.stored_int4
    ref = oattn.palu_decode_absorbed(store(lay["hk"]), store(lay["hv"]), qa, lens, s, 1, dh)
    err = rel_l2(got, ref)
    assert err.max() <= TOL, err.max()


def _tile_records(scores, chunk_tiles):
    """Per chunk of `chunk_tiles` 32-token tiles: the tile indices (within the chunk)
    whose maximum score exceeds every earlier tile's of that chunk."""
    tm = scores[: len(scores) // 32 * 32].reshape(-1, 32).max(axis=1)
    out = []
    for c in range(0, len(tm), chunk_tiles):
        seg = tm[c:c + chunk_tiles]
        run = np.maximum.accumulate(seg)
        out.append((np.nonzero(seg[1:] > run[:-1])[0] + 1, len(seg)))
    return out


@pytest.mark.parametrize("fmt_name,r,s,n_split", [("fp16", 256, 4, 1), ("fp16", 256, 4, 3), ("int4", 256, 4, 1),
                                                  ("int4", 256, 4, 2), ("int4", 64, 2, 1), ("fp16", 64, 2, 2)])
def test_absorbed_many_tiles_per_wave(fmt_name, r, s, n_split):
    """Each wave of the absorbed kernel walks tiles w, w + 4, ... of its chunk and
    carries its running max, running sum and accumulators from tile to tile. A
    forced small split count at T = 4096 gives every wave 8 to 32 tiles. The key
    latents' amplitude grows along the sequence, so that in every chunk of
    sequence 0 the running max moves at some tile past the first four (a record
    over the whole chunk is also a record of the wave owning that tile: the
    rescale of non-zero accumulators runs) and stays put at others (the
    unchanged-max branch runs). Sequence 1 is ragged, ending inside a chunk."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    B, T, U, dh = 2, 4096, 8, 128
    say(f"absorbed many tiles per wave: {fmt_name} r={r} heads/unit={s} T={T} n_split={n_split}")
    lay = synth.latent_layer(35, B, U, T, r, s * dh, 96.0)
    hk = lay["hk"] * np.linspace(0.4, 1.6, T, dtype=np.float32)[None, None, :, None]
    hv = lay["hv"]
    qa = synth.queries(36, B, U * s, r, 3.0)
    store = oattn.stored_fp16 if fmt == R.FMT_FP16 else oattn.stored_int4
    sk, sv = store(hk), store(hv)
    chunk_tiles = -(-(T // 32) // n_split)
    for j in range(U * s):
        for rec, n in _tile_records(sk[0, j // s] @ qa[0, j].astype(np.float64), chunk_tiles):
            assert (rec >= 4).any() and len(rec) < n - 1, (j, rec)
    cache = R.LatentCache(B, U, s, 1, dh, r, T, fmt, 0.0)
    cache.append(to_dev(hk), to_dev(hv))
    lens = np.array([T, T - 1013])
    cache.lens.copy_(torch.from_numpy(lens.astype(np.int32)))
    cache.host_lens[:] = lens
    got = cache.decode(R.MODE_ABSORBED, to_dev(qa), n_split=n_split)
    torch.cuda.synchronize()
    ref = oattn.palu_decode_absorbed(sk, sv, qa, lens, s, 1, dh)
    err = rel_l2(got.cpu().numpy(), ref)
    say(f"  max rel-L2 {err.max():.3g}")
    assert err.max() <= TOL, err.max()


@pytest.mark.parametrize("fmt_name", ["fp16", "int4"])
def test_absorbed_workload_sampled(fmt_name):
    """The absorbed-query workload at full size in the launch configuration the
    benchmark times: 16 sequences of 16K tokens, Llama-2-7B layer (8 units of 4
    heads, rank 256); the default chunking gives each (sequence, unit) 8 chunks of
    64 tiles, 16 tiles per wave. The cache is written on the device by torch from
    a seeded generator (fp16 latents sqrt(s_i) z; int4: random codes in [-7, 7]
    with decaying per-group scales); sampled (sequence, unit) pairs are read back
    and all four heads of each checked against the oracle."""
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    B, T, U, s, r, dh = 16, 16384, 8, 4, 256, 128
    say(f"absorbed workload sampled: {fmt_name} B={B} T={T}")
    dev = torch.device("cuda")
    g = torch.Generator(device=dev)
    g.manual_seed(37)
    cache = R.LatentCache(B, U, s, 1, dh, r, T, fmt, 0.0)
    root = torch.exp(-torch.arange(r, device=dev, dtype=torch.float32) / (2 * 96.0))
    if fmt == R.FMT_FP16:
        cache.hk.copy_((torch.randn(cache.hk.shape, generator=g, device=dev) * root).half())
        cache.hv.copy_((torch.randn(cache.hv.shape, generator=g, device=dev) * root[:, None]).half())
    else:
        for a in (cache.hk, cache.hv):
            c = torch.randint(-7, 8, a.shape[:-1] + (2 * a.shape[-1],), generator=g, device=dev, dtype=torch.int16)
            a.copy_(((c[..., 0::2] & 0xF) | ((c[..., 1::2] & 0xF) << 4)).to(torch.uint8))
        grp = root[16::32] / 4.0                                   # one scale per 32 ranks, ~ the group's amax / 7
        cache.sk.copy_((grp * (0.5 + torch.rand(cache.sk.shape, generator=g, device=dev))).half())
        cache.sv.copy_((grp[:, None] * (0.5 + torch.rand(cache.sv.shape, generator=g, device=dev))).half())
    cache.lens.fill_(T)
    cache.host_lens[:] = T
    qa = torch.randn((B, U * s, r), generator=g, device=dev) * 2.0
    got = cache.decode(R.MODE_ABSORBED, qa)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.isfinite(got).all()
    qn = qa.cpu().numpy()
    for b, u in ((0, 0), (9, 3), (15, 7)):
        if fmt == R.FMT_FP16:
            hk = cache.hk[b:b + 1, u:u + 1].cpu().numpy().astype(np.float64)
            hv = hv_fp16_tokens(cache.hv[b:b + 1, u:u + 1]).astype(np.float64)
        else:
            hk = hk_int4_codes(cache.hk[b:b + 1, u:u + 1]) * \
                np.repeat(cache.sk[b:b + 1, u:u + 1].cpu().numpy().astype(np.float64), 32, axis=-1)
            hv = hv_int4_codes(cache.hv[b:b + 1, u:u + 1]) * \
                np.repeat(sv_tokens(cache.sv[b:b + 1, u:u + 1]).astype(np.float64), 32, axis=-1)
        ref = oattn.palu_decode_absorbed(hk, hv, qn[b:b + 1, u * s:(u + 1) * s], [T], s, 1, dh)
        err = rel_l2(got[b, u * s:(u + 1) * s], ref[0]).max()
        say(f"  (b={b}, u={u}) max rel-L2 {err:.3g}")
        assert err <= TOL, ((b, u), err)


# ----------------------------------------------------------------------------- full size, sampled

def test_rope_full_size_sampled():
    """Llama-2-7B-shaped G-LRD layer at T = 64K in the bench's launch configuration;
    three query heads checked against the oracle one by one."""
    R = _R()
    T = 65536
    say(f"rope full size: llama2_glrd T={T} (sampled heads 0, 13, 31)")
    c = _make("llama2_glrd", T, T, R.FMT_FP16, seed=2)
    got = _gpu_rope(c)
    assert np.isfinite(got).all()
    for j in (0, 13, 31):
        u, w = oattn.head_unit(j, 4, 1)
        sub = dict(c)
        sub.update(q=c["q"][:, j:j + 1], sk=c["sk"][:, u:u + 1], sv=c["sv"][:, u:u + 1],
                   Bk=c["Bk"][u:u + 1, :, w * 128:(w + 1) * 128], s=1, gq=1)
        ref = _oracle_rope(sub)
        assert rel_l2(got[:, j], ref[:, 0]).max() <= TOL


def test_rope_gqa_full_size_sampled():
    """Llama-3-8B GQA shape, int4 latents, batch 4 at T = 64K in the bench's launch
    configuration; one query head of each KV head of sequences 0 and 3 checked
    against the oracle one by one."""
    R = _R()
    T, B = 65536, 4
    say(f"rope gqa full size: int4 B={B} T={T} (sampled heads)")
    U, s, gq, dh, r, th = 8, 1, 4, 128, 64, 5e5
    lay = synth.latent_layer(3, B, U, T, r, dh, 32.0)
    hk, Bk = synth.hadamard_mixed(lay["hk"], lay["Bk"])
    hv, _ = synth.hadamard_mixed(lay["hv"], lay["Bv"])
    q = synth.queries(1003, B, U * gq, dh, 1.0)
    cache = R.LatentCache(B, U, s, gq, dh, r, T, R.FMT_INT4_G32, th)
    cache.append(to_dev(hk), to_dev(hv))
    got = cache.decode(R.MODE_ROPE_RECON, to_dev(q), to_dev(Bk))
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    assert np.isfinite(got).all()
    lens = np.full(B, T, np.int64)
    for u in range(U):
        j = u * gq + (u % gq)
        for b in (0, 3):
            ref = oattn.palu_decode(oattn.stored_int4(hk[b:b + 1, u:u + 1]),
                                    oattn.stored_int4(hv[b:b + 1, u:u + 1]),
                                    Bk[u:u + 1].astype(np.float64), q[b:b + 1, j:j + 1], lens[:1],
                                    1, 1, dh, th)
            err = rel_l2(got[b:b + 1, j], ref[:, 0]).max()
            assert err <= TOL, (u, b, err)


def test_probe_stream_read_reads_every_word():
    """The streaming-read reference reads each 32-bit word exactly once: the XOR
    of its per-workgroup words equals the XOR of the buffer."""
    import rank_compressed_kv_amd as R
    say("stream-read probe")
    rng = np.random.default_rng(7)
    host = rng.integers(0, 2 ** 32, size=(1 << 20) + 4 * 37, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    for blocks in (1, 3, 64):
        out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
        R.probe_stream_read(buf, out, blocks)
        got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
        assert got == np.bitwise_xor.reduce(host), blocks
