"""A decode step (append of one token, then decode: prepare, partials, merge)
captured as a HIP graph and replayed must give what the same calls give eagerly:
three replays, each followed by eager work and a synchronisation, each compared
bit for bit with an identical cache stepped eagerly with the same host-side
length bound (so that both use the same chunking)."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import say, to_dev
from tests.test_gpu_latent import _R, _make

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,fmt_name,T,cap", [
    ("llama2_glrd", "fp16", 1000, 1056),     # config-2 kernel
    ("llama3_gqa", "int4", 777, 832),        # grouped-query int4 kernel
    ("tiny_glrd", "fp16", 200, 256),         # generic RoPE kernel
])
def test_graph_replay_matches_eager(name, fmt_name, T, cap):
    R = _R()
    fmt = R.FMT_FP16 if fmt_name == "fp16" else R.FMT_INT4_G32
    say(f"graph replay: {name} {fmt_name} T={T}")
    a = _make(name, T, cap, fmt, seed=41, mixed=fmt_name == "int4")
    b = _make(name, T, cap, fmt, seed=41, mixed=fmt_name == "int4")
    ca, cb = a["cache"], b["cache"]
    B, U, r = ca.B, ca.U, ca.r
    tok = synth.latent_layer(42, B, U, 1, r, a["s"] * a["dh"], 8.0)
    nk, nv = to_dev(tok["hk"]).contiguous(), to_dev(tok["hv"]).contiguous()
    q, bk = to_dev(a["q"]), to_dev(a["Bk"])
    bound = T + 8                               # host-side bound on every length reached
    mode = R.MODE_ROPE_RECON
    ws_a = torch.empty(R.decode_workspace_bytes(mode, ca.desc, bound), dtype=torch.uint8, device="cuda")
    ws_b = torch.empty_like(ws_a)
    out_a = torch.empty((B, q.shape[1], r), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    torch.cuda.synchronize()

    gph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gph):
        s = torch.cuda.current_stream()
        R.append_latent(mode, ca.desc, nk, nv, 1, bound - 1, stream=s)
        R.decode_attn(mode, ca.desc, q, bk, None, 0.0, out_a, ws_a, bound, stream=s)
    torch.cuda.synchronize()

    for rep in range(3):
        gph.replay()
        R.append_latent(mode, cb.desc, nk, nv, 1, bound - 1)
        R.decode_attn(mode, cb.desc, q, bk, None, 0.0, out_b, ws_b, bound)
        junk = torch.randn((512, 512), device="cuda") @ torch.randn((512, 512), device="cuda")
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
        la, lb = ca.lens.cpu().numpy(), cb.lens.cpu().numpy()
        assert np.array_equal(la, lb) and int(la[0]) == T + rep + 1, (la, lb)
        ga, gb = out_a.cpu().numpy(), out_b.cpu().numpy()
        assert np.isfinite(ga).all()
        assert np.array_equal(ga, gb), f"replay {rep}: max |diff| {np.abs(ga - gb).max()}"
