"""GPU parity of the projections on either side of the decode path (the cached
latents h = x A, and the output projection with B^v fused into W^o), through the
C ABI, against the float64 oracle; and one whole tiny layer x -> y."""
import numpy as np
import pytest
import torch

import synth
from oracle import attn as oattn
from oracle import prep as oprep
from tests.gpu_util import rel_l2, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import rank_compressed_kv_amd as R
    R.load_library()


def _R():
    import rank_compressed_kv_amd as R
    return R


@pytest.mark.parametrize("n_tok,d,U,r", [(1, 4096, 8, 256), (5, 4096, 8, 256), (16, 4096, 8, 256),
                                         (17, 96, 5, 16), (3, 4096, 8, 64)])
def test_latent_project_parity(n_tok, d, U, r):
    """h[t][u] = x_t A_u (Llama-2-7B G-LRD shape: d 4096, 8 units of rank 256)."""
    R = _R()
    say(f"latent projection: n_tok={n_tok} d={d} U={U} r={r}")
    rng = np.random.default_rng(70 + n_tok)
    x = rng.standard_normal((n_tok, d)).astype(np.float32)
    A = (rng.standard_normal((U, d, r)) / np.sqrt(d)).astype(np.float16)
    a_t = np.ascontiguousarray(np.transpose(A, (0, 2, 1)).reshape(U * r, d))
    h = R.latent_project(to_dev(x), to_dev(a_t), U, r).cpu().numpy()
    ref = oprep.latent_project(x, A.astype(np.float64))
    assert rel_l2(h.reshape(n_tok, -1), ref.reshape(n_tok, -1)).max() <= 1e-5


@pytest.mark.parametrize("B,Hq,r,d", [(1, 32, 256, 4096), (3, 32, 256, 4096), (16, 32, 256, 4096),
                                      (2, 4, 32, 256), (18, 3, 32, 48)])
def test_output_project_parity(B, Hq, r, d):
    """y = sum_j o_j (B^v_j W^o_j) (Llama-2-7B shape: 32 heads, rank 256, d 4096)."""
    R = _R()
    say(f"output projection: B={B} Hq={Hq} r={r} d={d}")
    rng = np.random.default_rng(80 + B)
    o = rng.standard_normal((B, Hq, r)).astype(np.float32)
    F = (rng.standard_normal((Hq, r, d)) / np.sqrt(Hq * r)).astype(np.float16)
    w_t = np.ascontiguousarray(F.reshape(Hq * r, d).T)
    y = R.output_project(to_dev(o), to_dev(w_t)).cpu().numpy()
    ref = np.stack([oattn.layer_output_fused(o[b], F.astype(np.float64)) for b in range(B)])
    assert rel_l2(y, ref).max() <= 1e-5


def test_projection_is_deterministic():
    R = _R()
    rng = np.random.default_rng(90)
    o = to_dev(rng.standard_normal((4, 32, 256)).astype(np.float32))
    w_t = to_dev((rng.standard_normal((4096, 32 * 256)) / 90).astype(np.float16))
    a = R.output_project(o, w_t).cpu().numpy()
    b = R.output_project(o, w_t).cpu().numpy()
    assert np.array_equal(a, b)


def test_tiny_layer_end_to_end():
    """Tiny G-LRD layer (d_model 256, 4 heads of 64, groups of 2, rank 32): tokens
    x -> latents (latent projection) -> cache (append) -> decode with RoPE ->
    layer output (fused output projection), against the oracle's float64 layer on
    the same fp16 weights."""
    R = _R()
    say("tiny layer end to end")
    tiny = synth.palu_tiny(seed=1)
    T, d, H, dh, s, r = 256, 256, 4, 64, 2, 32
    U = H // s
    root = np.sqrt(tiny["sv"][:r])
    # rank-r factors of the layer's K/V weights, from the factors they were built with
    Ak = (tiny["U_k"][:, :, :r] * root).astype(np.float16)                       # [U][d][r]
    Av = (tiny["U_v"][:, :, :r] * root).astype(np.float16)
    Bk = (root[:, None] * np.transpose(tiny["V_k"][:, :, :r], (0, 2, 1))).astype(np.float16)   # [U][r][s dh]
    Bv = root[:, None] * np.transpose(tiny["V_v"][:, :, :r], (0, 2, 1))
    # B^v_j W^o_j per head, rounded once to fp16
    F = np.stack([Bv[j // s][:, (j % s) * dh:(j % s + 1) * dh] @ tiny["W_o"][j * dh:(j + 1) * dh, :]
                  for j in range(H)]).astype(np.float16)                          # [H][r][d]
    x = tiny["x"].astype(np.float32)
    q = synth.queries(95, 1, H, dh, 1.5)

    hk = R.latent_project(to_dev(x), to_dev(np.ascontiguousarray(np.transpose(Ak, (0, 2, 1)).reshape(U * r, d))), U, r)
    hv = R.latent_project(to_dev(x), to_dev(np.ascontiguousarray(np.transpose(Av, (0, 2, 1)).reshape(U * r, d))), U, r)
    cache = R.LatentCache(1, U, s, 1, dh, r, T, R.FMT_FP16, 1e4)
    cache.append(hk.permute(1, 0, 2).unsqueeze(0).contiguous(), hv.permute(1, 0, 2).unsqueeze(0).contiguous())
    o = cache.decode(R.MODE_ROPE_RECON, to_dev(q), to_dev(Bk))
    y = R.output_project(o, to_dev(np.ascontiguousarray(F.reshape(H * r, d).T))).cpu().numpy()

    hk_ref = oprep.latent_project(x, Ak.astype(np.float64)).transpose(1, 0, 2)[None]
    hv_ref = oprep.latent_project(x, Av.astype(np.float64)).transpose(1, 0, 2)[None]
    o_ref = oattn.palu_decode(oattn.stored_fp16(hk_ref), oattn.stored_fp16(hv_ref), Bk.astype(np.float64), q,
                              [T], s, 1, dh, 1e4)
    y_ref = oattn.layer_output_fused(o_ref[0], F.astype(np.float64))
    assert rel_l2(y[0], y_ref) <= 2e-3
