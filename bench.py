#!/usr/bin/env python
"""Decode attention read directly from a low-rank latent KV cache, on one MI355X.

Default workload: one Llama-2-7B-shaped attention layer on the RoPE path
(d = 4096, 32 heads of 128, G-LRD groups of 4 heads -> 8 units, rank 256 per
unit = 50% of the K/V width, fp16 latents), batch 1, T = 65536 cached tokens.

One step = the whole decode hot path for one new token:
  append the token's K/V latents (fp32 -> fp16 cache)            lrkv_append_latent
  query preparation (rotated-basis queries)                      lrkv_decode_prepare
  latent stream + on-chip reconstruction + RoPE + online
  softmax + p.H^v, per sequence chunk                            lrkv_decode_partials
  split-K merge                                                  lrkv_merge_partials
Inputs are resident in HBM before the timed region. Two cache replicas are
used in turn so that consecutive steps do not re-read the same 537 MB from the
256 MB last-level cache.
The timed region holds the K steps and nothing else (no events inside it).

Prints one JSON line: the metric, whole-step throughput (latent-cache bytes per
second over the timed steps), the partials kernel's achieved bandwidth against
the HBM peak (roofline: the kernel's average launch duration over 20
back-to-back launches of the same workload; launches bracketed one by one in
an untimed diagnostic pass also appear under detail, inflated by the event
gaps), and the
float64 oracle timed on the host (cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "low-rank decode attn µs/step & latent-KV GB/s at T=64K; % of HBM peak"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0

# Llama-2-7B-shaped G-LRD layer
B, U, S, GQ, DH, R, THETA, TAU = 1, 8, 4, 1, 128, 256, 1e4, 96.0
BYTES_PER_UNIT_TOKEN = 2 * R * 2                      # K and V latents, fp16
FLOP_PER_UNIT_TOKEN = 2 * R * S * DH + 2 * S * DH + 2 * S * R


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


# the partials kernel's source and the headers it compiles in; their digest keys the
# recorded counter traffic
KERNEL_SOURCES = [os.path.join(ROOT, "rank_compressed_kv_amd", "csrc", f)
                  for f in ("rope_decode.hip", "tiles.h", "common.h")]
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "rope_decode_fw_llama2_7b_T65536.md")


def recorded_traffic():
    """HBM bytes per launch of the partials kernel from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy), or None when the kernel
    source or a header it includes has changed since they were taken."""
    import hashlib
    import re
    try:
        text = open(TRAFFIC_RECORD).read()
        h = hashlib.sha256()
        for f in KERNEL_SOURCES:
            h.update(open(f, "rb").read())
        src = h.hexdigest()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    t = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m or not t or m.group(1) != src:
        return None
    return float(t.group(1))


def _time(torch, fn, iters: int, warmup: int = 3) -> list:
    """Per-call GPU time (ms) of fn() from HIP events around each call."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def _row(ms: list, nbytes: float, flops: float = 0.0) -> dict:
    m = float(np.median(ms))
    out = {"us_median": round(m * 1e3, 2), "us_p10_p90": [round(float(np.percentile(ms, p)) * 1e3, 2) for p in (10, 90)],
           "algorithmic_bytes": nbytes, "GB_s": round(nbytes / (m * 1e-3) / 1e9, 1),
           "frac_hbm_peak": round(nbytes / (m * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if flops:
        out["tflops"] = round(flops / (m * 1e-3) / 1e12, 1)
    return out


def measure_stream_read(torch, lrkv, dev, nbytes: int = 4 << 30, iters: int = 10) -> dict:
    """The practical HBM read rate on this GPU: lrkv_probe_stream_read over a 4 GiB
    buffer (16x the last-level cache), median of `iters` launches."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    blocks = 8192
    out = torch.empty(blocks, dtype=torch.int32, device=dev)
    ms = _time(torch, lambda: lrkv.probe_stream_read(buf, out, blocks), iters)
    del buf, out
    m = float(np.median(ms))
    gbs = nbytes / (m * 1e-3) / 1e9
    return {"GB_s": round(gbs, 1), "bytes": nbytes, "us_median": round(m * 1e3, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def measure_rows(torch, lrkv, dev, iters: int = 20) -> dict:
    """The other hot-path rows at their workloads (one decode_attn call each, merge
    included; factorisation batches). Seeded synthetic inputs generated on the GPU:
    latents with the decaying spectrum sqrt(s_i) z, low-rank-plus-noise paged K/V."""
    g = torch.Generator(device=dev)
    rows = {}

    # absorbed (no RoPE) over fp16 latents: Llama-2-7B layer, 16 sequences of 16K
    g.manual_seed(3)
    Bq, Tq = 16, 16384
    c = lrkv.LatentCache(Bq, U, S, GQ, DH, R, Tq, lrkv.FMT_FP16, 0.0, device=dev)
    sq = torch.exp(-torch.arange(R, device=dev, dtype=torch.float32) / (2 * TAU))
    c.hk.copy_((torch.randn(c.hk.shape, generator=g, device=dev) * sq).half())
    c.hv.copy_((torch.randn(c.hv.shape, generator=g, device=dev) * sq[:, None]).half())
    c.lens.fill_(Tq)
    c.host_lens[:] = Tq
    qa = torch.randn((Bq, U * S * GQ, R), generator=g, device=dev) * 0.35
    ws = c.workspace(lrkv.MODE_ABSORBED)
    out = torch.empty((Bq, U * S * GQ, R), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda: lrkv.decode_attn(lrkv.MODE_ABSORBED, c.desc, qa, None, None, 0.0, out, ws, Tq), iters)
    rows["absorbed_fp16_B16_T16384"] = _row(ms, Bq * U * Tq * BYTES_PER_UNIT_TOKEN, Bq * U * Tq * 4 * S * R)
    del c, ws

    # absorbed over int4 latents (symmetric codes, one fp16 scale per 32 elements
    # per token), same layer and batch: codes + scales are 288 B per unit-token
    c = lrkv.LatentCache(Bq, U, S, GQ, DH, R, Tq, lrkv.FMT_INT4_G32, 0.0, device=dev)
    for chunk in range(0, Tq, 4096):
        c.append(torch.randn((Bq, U, 4096, R), generator=g, device=dev) * sq,
                 torch.randn((Bq, U, 4096, R), generator=g, device=dev) * sq)
    ws = c.workspace(lrkv.MODE_ABSORBED)
    ms = _time(torch, lambda: lrkv.decode_attn(lrkv.MODE_ABSORBED, c.desc, qa, None, None, 0.0, out, ws, Tq), iters)
    rows["absorbed_int4_B16_T16384"] = _row(ms, Bq * U * Tq * 2 * (R // 2 + 2 * R // 32), Bq * U * Tq * 4 * S * R)
    del c, qa, ws, out

    # the RoPE path of the same layer at the sweep's shorter lengths (B = 1, one
    # decode_attn call: prepare, partials, merge); T = 64K is the main line
    g.manual_seed(7)
    Ts = 32768
    c = lrkv.LatentCache(1, U, S, GQ, DH, R, Ts, lrkv.FMT_FP16, THETA, device=dev)
    c.hk.copy_((torch.randn(c.hk.shape, generator=g, device=dev) * sq).half())
    c.hv.copy_((torch.randn(c.hv.shape, generator=g, device=dev) * sq[:, None]).half())
    q2 = torch.randn((1, U * S * GQ, DH), generator=g, device=dev)
    bk2 = (torch.randn((U, R, S * DH), generator=g, device=dev) / 16.0).half()
    out = torch.empty((1, U * S * GQ, R), dtype=torch.float32, device=dev)
    for Tn in (4096, 16384, 32768):
        c.lens.fill_(Tn)
        c.host_lens[:] = Tn
        ws = c.workspace(lrkv.MODE_ROPE_RECON)
        ms = _time(torch, lambda: lrkv.decode_attn(lrkv.MODE_ROPE_RECON, c.desc, q2, bk2, None, 0.0, out, ws, Tn),
                   iters)
        rows[f"rope_fp16_B1_T{Tn}"] = _row(ms, U * Tn * BYTES_PER_UNIT_TOKEN, U * Tn * FLOP_PER_UNIT_TOKEN)
    del c, ws, out, q2, bk2

    # the projections on either side of the path (Llama-2-7B layer): latents of K and V
    # for a new token of every sequence (one call, 16 units of rank 256, d 4096) and
    # the output projection with B^v fused into W^o (32 heads x 256 -> 4096); fp16
    # weights streamed once per call
    g.manual_seed(6)
    DM = U * S * DH
    a_t = (torch.randn((2 * U * R, DM), generator=g, device=dev) / DM ** 0.5).half()
    w_t = (torch.randn((DM, U * S * R), generator=g, device=dev) / (U * S * R) ** 0.5).half()
    for nb in (1, 16):
        x = torch.randn((nb, DM), generator=g, device=dev)
        o = torch.randn((nb, U * S, R), generator=g, device=dev)
        h = torch.empty((nb, 2 * U, R), dtype=torch.float32, device=dev)
        y = torch.empty((nb, DM), dtype=torch.float32, device=dev)
        wsl = torch.empty(lrkv.project_workspace_bytes(nb, 2 * U * R, DM), dtype=torch.uint8, device=dev)
        wso = torch.empty(lrkv.project_workspace_bytes(nb, DM, U * S * R), dtype=torch.uint8, device=dev)
        ms = _time(torch, lambda: lrkv.latent_project(x, a_t, 2 * U, R, h, wsl), iters)
        rows[f"latent_project_kv_B{nb}"] = _row(ms, a_t.numel() * 2, 2 * nb * a_t.numel())
        ms = _time(torch, lambda: lrkv.output_project(o, w_t, y, wso), iters)
        rows[f"output_project_B{nb}"] = _row(ms, w_t.numel() * 2, 2 * nb * w_t.numel())
    del a_t, w_t, x, o, h, y, wsl, wso

    # chunked prefill on the RoPE path: Llama-2-7B layer, a 512-token chunk appended
    # at position 65024 attends causally over the 64K-token latent cache. Algorithmic
    # work: the reconstruction once per (token, head) plus scores and values per
    # (query, visible token); the kernel redoes the reconstruction per 64-query block
    # and forms scores from fp16 hi + lo parts (more MFMA work than counted)
    g.manual_seed(7)
    Tp, Mp = 65536, 512
    c = lrkv.LatentCache(1, U, S, GQ, DH, R, Tp, lrkv.FMT_FP16, THETA, device=dev)
    sq = torch.exp(-torch.arange(R, device=dev, dtype=torch.float32) / (2 * TAU))
    for t0 in range(0, Tp, 16384):
        c.append(torch.randn((1, U, 16384, R), generator=g, device=dev) * sq,
                 torch.randn((1, U, 16384, R), generator=g, device=dev) * sq)
    qp = torch.randn((1, Mp, U * S * GQ, DH), generator=g, device=dev)
    bkp = (torch.randn((U, R, S * DH), generator=g, device=dev) / 16).half()
    p0 = torch.full((1,), Tp - Mp, dtype=torch.int32, device=dev)
    wsp = c.prefill_workspace(Mp)
    outp = torch.empty((1, Mp, U * S * GQ, R), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda: c.prefill_attn(qp, bkp, p0, out=outp, workspace=wsp), 10)
    heads = U * S * GQ
    vis = float(sum(Tp - Mp + m + 1 for m in range(Mp)))
    flops_p = 2.0 * R * DH * Tp * heads + 2.0 * (DH + R) * vis * heads
    rows["prefill_chunk512_T65536"] = _row(ms, U * Tp * 2 * R * 2, flops_p)
    rows["prefill_chunk512_T65536"]["frac_mfma_peak"] = round(flops_p / (float(np.median(ms)) * 1e-3) / 1e12
                                                             / MFMA_F16_PEAK_TFLOPS, 4)
    del c, qp, bkp, p0, wsp, outp

    # RoPE path over Hadamard-rotated int4 latents: Llama-3-8B GQA, rank 64 per KV head
    g.manual_seed(4)
    B4, T4, H4, G4, R4 = 4, 65536, 8, 4, 64
    c = lrkv.LatentCache(B4, H4, 1, G4, DH, R4, T4, lrkv.FMT_INT4_G32, 5e5, device=dev)
    s4 = torch.exp(-torch.arange(R4, device=dev, dtype=torch.float32) / 64.0)
    for chunk in range(0, T4, 16384):
        hk = torch.randn((B4, H4, 16384, R4), generator=g, device=dev) * s4
        hv = torch.randn((B4, H4, 16384, R4), generator=g, device=dev) * s4
        c.append(hk, hv)
    q4 = torch.randn((B4, H4 * G4, DH), generator=g, device=dev)
    bk4 = (torch.randn((H4, R4, DH), generator=g, device=dev) / 8.0).half()
    ws = c.workspace(lrkv.MODE_ROPE_RECON)
    out = torch.empty((B4, H4 * G4, R4), dtype=torch.float32, device=dev)
    ms = _time(torch, lambda: lrkv.decode_attn(lrkv.MODE_ROPE_RECON, c.desc, q4, bk4, None, 0.0, out, ws, T4), iters)
    rows["rope_int4_gqa_B4_T65536"] = _row(ms, B4 * H4 * T4 * 72, B4 * H4 * T4 * (2 * R4 * DH + 2 * G4 * DH + 2 * G4 * R4))
    del c, q4, bk4, ws, out, hk, hv

    # PuzzleKV hybrid: Llama-3.1-8B shape, batch 8, T = 32K, rank-12 pages
    g.manual_seed(5)
    B5, H5, G5, T5, P5, RK = 8, 8, 4, 32768, 32, 12
    pc = lrkv.PagedCache(B5, H5, G5, DH, P5, 1, 4, RK, RK, T5 // P5 + 8, device=dev)
    def lowrank():
        z = torch.randn((B5 * H5, T5, RK), generator=g, device=dev)
        cm = torch.randn((B5 * H5, RK, DH), generator=g, device=dev) / RK ** 0.5
        x = torch.bmm(z, cm) + 0.05 * torch.randn((B5 * H5, T5, DH), generator=g, device=dev)
        return x.view(B5, H5, T5, DH).half()
    k5, v5 = lowrank(), lowrank()
    pages = torch.from_numpy(lrkv.paged_plan(pc.desc, pc.host_lens, T5)).to(dev)
    n_fac = int(pages.shape[0])
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    lrkv.factor_page(pc.desc, pages, n_fac, k5, v5, T5, 0)
    t1.record()
    lrkv.append_latent(lrkv.MODE_HYBRID_PAGED, pc.desc, k5, v5, T5, 0)
    pc.host_lens += T5
    torch.cuda.synchronize()
    prefill_ms = t0.elapsed_time(t1)
    q5 = torch.randn((B5, H5 * G5, DH), generator=g, device=dev)
    ws = pc.workspace()
    out = torch.empty((B5, H5 * G5, DH), dtype=torch.float32, device=dev)
    n_dense, n_factored = 5, T5 // P5 - 5
    by = B5 * H5 * (n_factored * 2 * (P5 * RK + RK * DH) * 2 + n_dense * 2 * P5 * DH * 2)
    ms = _time(torch, lambda: pc.decode(q5, out=out, workspace=ws), iters)
    rows["hybrid_paged_B8_T32768"] = _row(ms, by)
    # one decode step's factorisation batch: one page per (b, head), keys and values
    step_pages = pages.view(B5, H5, -1, 3)[:, :, -1, :].reshape(-1, 3).contiguous()
    ms = _time(torch, lambda: lrkv.factor_page(pc.desc, step_pages, step_pages.shape[0], k5, v5, T5, 0), iters)
    rows["factor_pages_decode_batch"] = {"matrices": 2 * int(step_pages.shape[0]),
                                         "us_median": round(float(np.median(ms)) * 1e3, 2)}
    rows["factor_pages_prefill_batch"] = {"matrices": 2 * n_fac, "us": round(prefill_ms * 1e3, 1)}
    del pc, ws

    # the same cache with int4 page factors (one fp16 scale per 32 stored elements):
    # codes + scales are (P r + r d) (1/2 + 2/32) bytes per factor pair
    pc4 = lrkv.PagedCache(B5, H5, G5, DH, P5, 1, 4, RK, RK, T5 // P5 + 8, device=dev,
                          factor_fmt=lrkv.FMT_INT4_G32)
    lrkv.factor_page(pc4.desc, pages, n_fac, k5, v5, T5, 0)
    lrkv.append_latent(lrkv.MODE_HYBRID_PAGED, pc4.desc, k5, v5, T5, 0)
    pc4.host_lens += T5
    torch.cuda.synchronize()
    ws = pc4.workspace()
    per_side = (P5 * RK + RK * DH) // 2 + (P5 * RK + RK * DH) // 32 * 2
    by4 = B5 * H5 * (n_factored * 2 * per_side + n_dense * 2 * P5 * DH * 2)
    ms = _time(torch, lambda: pc4.decode(q5, out=out, workspace=ws), iters)
    rows["hybrid_paged_int4_B8_T32768"] = _row(ms, by4)
    del pc4, ws, k5, v5
    return rows


def cpu_baseline(T: int, budget_s: float = 12.0) -> dict:
    """The float64 oracle timed on this host on a bounded sample of the same workload:
    whole units (4 heads each) at full length, until the time budget is used."""
    import synth
    from oracle import attn as oattn
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    lay = synth.latent_layer(2, 1, 1, T, R, S * DH, TAU)
    q = synth.queries(1002, 1, S * GQ, DH)
    hk = oattn.stored_fp16(lay["hk"])
    hv = oattn.stored_fp16(lay["hv"])
    Bk = lay["Bk"].astype(np.float64)
    units, elapsed = 0, 0.0
    while elapsed < budget_s and units < U:
        t0 = time.perf_counter()
        oattn.palu_decode(hk, hv, Bk, q, [T], S, GQ, DH, THETA)
        elapsed += time.perf_counter() - t0
        units += 1
    gbs = units * T * BYTES_PER_UNIT_TOKEN / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{units} of {U} units (4 query heads each) at T={T}, float64 numpy oracle, "
                      f"{elapsed:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--T", type=int, default=65536)
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the timing of the other hot-path rows (absorbed, int4, hybrid, factorisation)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU and has no multi-GPU path (the decode would "
              "shard by unit, batch or sequence chunk, exchanging only the per-chunk "
              "partial states before the merge)", file=sys.stderr)
        return 2

    import torch

    import rank_compressed_kv_amd as lrkv
    import synth

    lrkv.load_library()
    dev = torch.device("cuda:0")
    T, K, W, NR, D = args.T, args.steps, args.warmup, max(1, args.replicas), 8
    T_init = T - 1 - W // NR
    cap = ((T + K + W + D + 64) // 32) * 32

    log(f"bench: generating latents for T={T_init} (B={B}, U={U}, r={R})")
    lay = synth.latent_layer(2, B, U, T_init, R, S * DH, TAU)
    hk0 = torch.from_numpy(lay["hk"]).to(dev)
    hv0 = torch.from_numpy(lay["hv"]).to(dev)
    Bk = torch.from_numpy(lay["Bk"]).to(dev)
    del lay
    reps = []
    for i in range(NR):
        c = lrkv.LatentCache(B, U, S, GQ, DH, R, cap, lrkv.FMT_FP16, THETA, device=dev)
        c.append(hk0, hv0)
        reps.append(c)
    del hk0, hv0
    step_tok = synth.latent_layer(3, B, U, W + K + D, R, S * DH, TAU)
    nk = torch.from_numpy(step_tok["hk"]).to(dev)
    nv = torch.from_numpy(step_tok["hv"]).to(dev)
    new_k = [nk[:, :, i:i + 1].contiguous() for i in range(W + K + D)]
    new_v = [nv[:, :, i:i + 1].contiguous() for i in range(W + K + D)]
    q = torch.from_numpy(synth.queries(1002, B, U * S * GQ, DH)).to(dev)
    out = torch.empty((B, U * S * GQ, R), dtype=torch.float32, device=dev)
    for c in reps:          # the workspace must cover the longest length of the run
        c.host_lens += K + W + D
    ws = [c.workspace(lrkv.MODE_ROPE_RECON, args.n_split) for c in reps]
    for c in reps:
        c.host_lens -= K + W + D
    torch.cuda.synchronize()

    if args.copy_probe:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    mode = lrkv.MODE_ROPE_RECON
    stream = torch.cuda.current_stream()

    def step(i: int, ev=None) -> int:
        """One decode step on replica i % NR; ev = events to record around its phases
        (2: the partials kernel only; 5: every phase)."""
        c, w = reps[i % NR], ws[i % NR]
        if ev is not None and len(ev) == 5:
            ev[0].record()
        c.append(new_k[i], new_v[i], stream=stream)
        L = c.max_len
        if ev is not None and len(ev) == 5:
            ev[1].record()
        lrkv.decode_prepare(mode, c.desc, q, Bk, None, 0.0, w, L, args.n_split, stream=stream)
        if ev is not None:
            ev[-3 if len(ev) == 5 else 0].record()
        lrkv.decode_partials(mode, c.desc, None, 0.0, w, L, args.n_split, stream=stream)
        if ev is not None:
            ev[-2 if len(ev) == 5 else 1].record()
        lrkv.merge_partials(mode, c.desc, out, w, L, args.n_split, stream=stream)
        if ev is not None and len(ev) == 5:
            ev[4].record()
        return L

    mk = lambda n: [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    # timed region: K whole steps, no events inside (a recorded event costs the
    # GPU several microseconds)
    t_start, t_end = mk(2)
    log(f"bench: {W} warmup + {K} timed steps, {NR} cache replicas")
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    t_start.record()
    h0 = time.perf_counter()
    lens_timed = [step(W + k) for k in range(K)]
    host_us = (time.perf_counter() - h0) / K * 1e6
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    # untimed diagnostic pass: every phase bracketed by events
    dev_ev = [mk(5) for _ in range(D)]
    for k in range(D):
        step(W + K + k, dev_ev[k])
    torch.cuda.synchronize()
    ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in dev_ev])
    part_each = ph[:, 2]           # the partials kernel of each diagnostic step
    # the kernel's average launch duration: NB back-to-back partials launches of the
    # timed workload (the replicas in turn, at their current lengths), one event
    # pair around the batch, so that no per-launch event gap enters the average
    NB = 20
    b0, b1 = mk(2)
    lens_b = [reps[k % NR].max_len for k in range(NB)]
    b0.record()
    for k in range(NB):
        lrkv.decode_partials(mode, reps[k % NR].desc, None, 0.0, ws[k % NR], lens_b[k], args.n_split, stream=stream)
    b1.record()
    torch.cuda.synchronize()
    part_batch_ms = b0.elapsed_time(b1) / NB

    lens_timed = np.array(lens_timed, dtype=np.float64)
    bytes_steps = U * B * lens_timed * BYTES_PER_UNIT_TOKEN
    flops_steps = U * B * lens_timed * FLOP_PER_UNIT_TOKEN
    gbs = bytes_steps.sum() / (total_ms * 1e-3) / 1e9
    part_ms = part_each.mean()
    achieved = U * B * float(np.mean(lens_b)) * BYTES_PER_UNIT_TOKEN / (part_batch_ms * 1e-3) / 1e9
    ok = bool(np.isfinite(out.cpu().numpy()).all())
    traffic = recorded_traffic()

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(total_ms / K, 5),
        "us_per_step": round(total_ms / K * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "Llama-2-7B-shaped G-LRD attention layer, RoPE reconstruct path, "
                        "8 units x 4 heads, d_h 128, rank 256 per unit, fp16 latents",
            "batch": B, "T": T, "T_mean_timed": float(lens_timed.mean()), "units": U,
            "heads": U * S * GQ, "rank": R, "head_dim": DH, "rope_theta": THETA,
            "cache_replicas": NR, "n_split": args.n_split,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "rope_decode (lrkv_decode_partials)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "detail": {
            "phase_us_untimed_pass": {"append": round(ph[:, 0].mean() * 1e3, 2),
                                      "prepare": round(ph[:, 1].mean() * 1e3, 2),
                                      "partials": round(ph[:, 2].mean() * 1e3, 2),
                                      "merge": round(ph[:, 3].mean() * 1e3, 2)},
            "partials_us_batch_avg": round(part_batch_ms * 1e3, 2),
            "partials_us_mean_p10_p50_p90": [round(part_ms * 1e3, 2)] +
                                            [round(float(np.percentile(part_each, p)) * 1e3, 2) for p in (10, 50, 90)],
            "mfma_tflops_partials": round(flops_steps.mean() / (part_batch_ms * 1e-3) / 1e12, 1),
            "mfma_frac_partials": round(flops_steps.mean() / (part_batch_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "bytes_per_step": float(bytes_steps.mean()),
            "host_submit_us_per_step": round(host_us, 1),
            "output_finite": ok,
        },
    }
    del reps, ws
    torch.cuda.empty_cache()
    log("bench: streaming-read reference")
    sr = measure_stream_read(torch, lrkv, dev)
    result["detail"]["stream_read"] = sr
    result["detail"]["partials_frac_stream_read"] = round(achieved / sr["GB_s"], 4)
    if not args.no_rows:
        log("bench: timing the other hot-path rows")
        rows = measure_rows(torch, lrkv, dev)
        for r in rows.values():
            if "GB_s" in r:
                r["frac_stream_read"] = round(r["GB_s"] / sr["GB_s"], 4)
        result["detail"]["rows"] = rows
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline(T)
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
