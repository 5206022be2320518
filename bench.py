#!/usr/bin/env python
"""Decode attention read directly from a low-rank latent KV cache, on one MI355X.

Default workload: one Llama-2-7B-shaped attention layer on the RoPE path
(d = 4096, 32 heads of 128, G-LRD groups of 4 heads -> 8 units, rank 256 per
unit = 50% of the K/V width, fp16 latents), batch 1, T = 65536 cached tokens.

One step = the whole decode hot path for one new token, one lrkv_decode_step
call (three launches):
  query preparation (rotated-basis queries, RoPE angle tables)
    with the append of the token's K/V latents (fp32 -> fp16)     rope_prepare
  latent stream + on-chip reconstruction + RoPE + online
  softmax + p.H^v, per sequence chunk                             rope_decode_fw
  split-K merge, and the lengths advance                          merge_splits
The untimed passes that bracket kernels with events issue the same work as the
four calls lrkv_append_latent, lrkv_decode_prepare, lrkv_decode_partials and
lrkv_merge_partials.
Inputs are resident in HBM before the timed region. Two cache replicas are
used in turn so that consecutive steps do not re-read the same 537 MB from the
256 MB last-level cache. The timed region holds the K steps and nothing else
(no events inside it).

Prints one JSON line: the metric, whole-step throughput (latent-cache bytes per
second over the timed steps), the partials kernel's achieved bandwidth against
the HBM peak (roofline: the kernel's mean duration inside decode steps, from
events around that kernel alone in an untimed pass of whole steps run right
after the timed region), the other hot-path rows with cold-cache figures
(replicas rotated so that each call reads from HBM) beside warm ones, and the
float64 oracle timed on the host (cpu_baseline) at one thread and at all cores.

`python bench.py --trace-summary <kernel_trace.csv> --steps K --warmup W`
reads a rocprofv3 kernel trace of a bench run with the same K and W and prints
the per-step statistics of the timed steps (duration of each kernel, whole step
from the first kernel's start to the last one's end: mean, p10, p50, p90), and the
partials kernel's mean over the untimed pass whose events feed roofline.achieved.
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
COLD_BYTES = 1 << 30          # replicas of a row's cache add up to at least this (4x the last-level cache)

# Llama-2-7B-shaped G-LRD layer
B, U, S, GQ, DH, R, THETA, TAU = 1, 8, 4, 1, 128, 256, 1e4, 96.0
BYTES_PER_UNIT_TOKEN = 2 * R * 2                      # K and V latents, fp16
FLOP_PER_UNIT_TOKEN = 2 * R * S * DH + 2 * S * DH + 2 * S * R

# kernels of one decode step, in launch order (names as the kernel trace shows them):
# lrkv_decode_step, and the same step issued as four calls
STEP_KERNELS = ("rope_prepare", "rope_decode_fw", "merge_splits")
SPLIT_STEP_KERNELS = ("append_fp16_small", "rope_prepare", "rope_decode_fw", "merge_splits")


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


def _pct(a, ps=(10, 50, 90)):
    return [round(float(np.percentile(a, p)), 2) for p in ps]


# ----------------------------------------------------------------------------- row timing

def _batch_us(torch, fns, n: int) -> float:
    """Mean GPU time (us) per call of n calls cycling through `fns`, one event pair
    around the whole batch (no per-call event gaps)."""
    for f in fns[:3]:
        f()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(n):
        fns[i % len(fns)]()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e3


def _each_us(torch, fns, n: int) -> list:
    """Per-call GPU time (us) from an event pair around each call (adds the event gaps)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(ev):
        a.record()
        fns[i % len(fns)]()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) * 1e3 for a, b in ev]


def _row(torch, fns, nbytes: float, flops: float = 0.0, n: int = 200, replica_bytes: float = 0.0) -> dict:
    """Cold figure: calls cycling through the replicas (each call's data comes from
    HBM); warm figure: the same calls on the first replica only."""
    cold = _batch_us(torch, fns, n)
    warm = _batch_us(torch, fns[:1], n)
    each = _each_us(torch, fns, max(40, len(fns)))
    out = {"us_cold": round(cold, 2), "us_warm": round(warm, 2),
           "us_cold_each_p10_p50_p90": _pct(each), "replicas": len(fns),
           "replica_bytes": replica_bytes or nbytes, "algorithmic_bytes": nbytes,
           "GB_s": round(nbytes / (cold * 1e-6) / 1e9, 1),
           "GB_s_warm": round(nbytes / (warm * 1e-6) / 1e9, 1),
           "frac_hbm_peak": round(nbytes / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
           "frac_hbm_peak_warm": round(nbytes / (warm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
    if flops:
        out["tflops"] = round(flops / (cold * 1e-6) / 1e12, 1)
    return out


def _n_replicas(nbytes: float) -> int:
    return max(1, int(np.ceil(COLD_BYTES / nbytes)))


def measure_stream_read(torch, lrkv, dev, nbytes: int = 4 << 30, iters: int = 10) -> dict:
    """The practical HBM read rate on this GPU: lrkv_probe_stream_read over a 4 GiB
    buffer (16x the last-level cache), median of `iters` launches."""
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    blocks = 8192
    out = torch.empty(blocks, dtype=torch.int32, device=dev)
    ms = _each_us(torch, [lambda: lrkv.probe_stream_read(buf, out, blocks)], iters)
    del buf, out
    m = float(np.median(ms))
    gbs = nbytes / (m * 1e-6) / 1e9
    return {"GB_s": round(gbs, 1), "bytes": nbytes, "us_median": round(m, 1),
            "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}


def _latent_replicas(torch, lrkv, c, n: int) -> list:
    """n caches holding the same contents as c (c itself first)."""
    reps = [c]
    for _ in range(n - 1):
        d = lrkv.LatentCache(c.B, c.U, c.s, c.gq, c.dh, c.r, c.cap, c.fmt, c.theta, device=c.hk.device)
        for name in ("hk", "hv", "sk", "sv", "lens"):
            if getattr(c, name) is not None:
                getattr(d, name).copy_(getattr(c, name))
        d.host_lens[:] = c.host_lens
        reps.append(d)
    return reps


def _paged_replicas(torch, lrkv, c, n: int) -> list:
    reps = [c]
    for _ in range(n - 1):
        d = lrkv.PagedCache(c.B, c.H, c.G, c.d, c.P, c.sink, c.window, c.rk_, c.rv_, c.max_pages,
                            device=c.dense_k.device, factor_fmt=c.factor_fmt)
        for name in ("dense_k", "dense_v", "lk", "rk", "lv", "rv", "lk_s", "rk_s", "lv_s", "rv_s",
                     "page_table", "lens"):
            if getattr(c, name) is not None:
                getattr(d, name).copy_(getattr(c, name))
        d.host_lens[:] = c.host_lens
        reps.append(d)
    return reps


def _latent_bytes(c) -> float:
    return float(sum(t.numel() * t.element_size() for t in (c.hk, c.hv, c.sk, c.sv) if t is not None))


def measure_rows(torch, lrkv, dev) -> dict:
    """The other hot-path rows at their workloads (one decode_attn call each, merge
    included; factorisation batches), cold-cache (replicas of the row's cache adding up
    to >= 1 GiB, called in turn) and warm. Seeded synthetic inputs generated on the
    GPU: latents with the decaying spectrum sqrt(s_i) z, low-rank-plus-noise paged K/V."""
    g = torch.Generator(device=dev)
    rows = {}
    sq = torch.exp(-torch.arange(R, device=dev, dtype=torch.float32) / (2 * TAU))

    # absorbed (no RoPE) over fp16 latents: Llama-2-7B layer, 16 sequences of 16K
    g.manual_seed(3)
    Bq, Tq = 16, 16384
    c = lrkv.LatentCache(Bq, U, S, GQ, DH, R, Tq, lrkv.FMT_FP16, 0.0, device=dev)
    c.hk.copy_((torch.randn(c.hk.shape, generator=g, device=dev) * sq).half())
    c.hv.copy_((torch.randn(c.hv.shape, generator=g, device=dev) * sq[:, None]).half())
    c.lens.fill_(Tq)
    c.host_lens[:] = Tq
    qa = torch.randn((Bq, U * S * GQ, R), generator=g, device=dev) * 0.35
    out = torch.empty((Bq, U * S * GQ, R), dtype=torch.float32, device=dev)
    nb = Bq * U * Tq * BYTES_PER_UNIT_TOKEN
    reps = _latent_replicas(torch, lrkv, c, _n_replicas(_latent_bytes(c)))
    wss = [r.workspace(lrkv.MODE_ABSORBED) for r in reps]
    fns = [lambda r=r, w=w: lrkv.decode_attn(lrkv.MODE_ABSORBED, r.desc, qa, None, None, 0.0, out, w, Tq)
           for r, w in zip(reps, wss)]
    rows["absorbed_fp16_B16_T16384"] = _row(torch, fns, nb, Bq * U * Tq * 4 * S * R, replica_bytes=_latent_bytes(c))
    del c, reps, wss, fns

    # absorbed over int4 latents (symmetric codes, one fp16 scale per 32 elements
    # per token), same layer and batch: codes + scales are 288 B per unit-token
    c = lrkv.LatentCache(Bq, U, S, GQ, DH, R, Tq, lrkv.FMT_INT4_G32, 0.0, device=dev)
    for chunk in range(0, Tq, 4096):
        c.append(torch.randn((Bq, U, 4096, R), generator=g, device=dev) * sq,
                 torch.randn((Bq, U, 4096, R), generator=g, device=dev) * sq)
    nb = Bq * U * Tq * 2 * (R // 2 + 2 * R // 32)
    reps = _latent_replicas(torch, lrkv, c, _n_replicas(_latent_bytes(c)))
    wss = [r.workspace(lrkv.MODE_ABSORBED) for r in reps]
    fns = [lambda r=r, w=w: lrkv.decode_attn(lrkv.MODE_ABSORBED, r.desc, qa, None, None, 0.0, out, w, Tq)
           for r, w in zip(reps, wss)]
    rows["absorbed_int4_B16_T16384"] = _row(torch, fns, nb, Bq * U * Tq * 4 * S * R, replica_bytes=_latent_bytes(c))
    del c, reps, wss, fns, qa, out

    # the RoPE path of the same layer at the sweep's shorter lengths (B = 1, one
    # decode_attn call: prepare, partials, merge); T = 64K is the main line
    g.manual_seed(7)
    q2 = torch.randn((1, U * S * GQ, DH), generator=g, device=dev)
    bk2 = (torch.randn((U, R, S * DH), generator=g, device=dev) / 16.0).half()
    out = torch.empty((1, U * S * GQ, R), dtype=torch.float32, device=dev)
    for Tn in (4096, 16384, 32768):
        c = lrkv.LatentCache(1, U, S, GQ, DH, R, Tn, lrkv.FMT_FP16, THETA, device=dev)
        c.hk.copy_((torch.randn(c.hk.shape, generator=g, device=dev) * sq).half())
        c.hv.copy_((torch.randn(c.hv.shape, generator=g, device=dev) * sq[:, None]).half())
        c.lens.fill_(Tn)
        c.host_lens[:] = Tn
        reps = _latent_replicas(torch, lrkv, c, _n_replicas(_latent_bytes(c)))
        wss = [r.workspace(lrkv.MODE_ROPE_RECON) for r in reps]
        fns = [lambda r=r, w=w, Tn=Tn: lrkv.decode_attn(lrkv.MODE_ROPE_RECON, r.desc, q2, bk2, None, 0.0, out, w, Tn)
               for r, w in zip(reps, wss)]
        rows[f"rope_fp16_B1_T{Tn}"] = _row(torch, fns, U * Tn * BYTES_PER_UNIT_TOKEN, U * Tn * FLOP_PER_UNIT_TOKEN,
                                           replica_bytes=_latent_bytes(c))
        del c, reps, wss, fns
    del q2, bk2, out

    # the projections on either side of the path (Llama-2-7B layer): latents of K and V
    # for a new token of every sequence (one call, 16 units of rank 256, d 4096) and
    # the output projection with B^v fused into W^o (32 heads x 256 -> 4096); fp16
    # weights streamed once per call, replicas of the weights for the cold figure
    g.manual_seed(6)
    DM = U * S * DH
    a_t = (torch.randn((2 * U * R, DM), generator=g, device=dev) / DM ** 0.5).half()
    w_t = (torch.randn((DM, U * S * R), generator=g, device=dev) / (U * S * R) ** 0.5).half()
    a_reps = [a_t] + [a_t.clone() for _ in range(_n_replicas(a_t.numel() * 2) - 1)]
    w_reps = [w_t] + [w_t.clone() for _ in range(_n_replicas(w_t.numel() * 2) - 1)]
    for nbt in (1, 16):
        x = torch.randn((nbt, DM), generator=g, device=dev)
        o = torch.randn((nbt, U * S, R), generator=g, device=dev)
        h = torch.empty((nbt, 2 * U, R), dtype=torch.float32, device=dev)
        y = torch.empty((nbt, DM), dtype=torch.float32, device=dev)
        wsl = torch.empty(lrkv.project_workspace_bytes(nbt, 2 * U * R, DM), dtype=torch.uint8, device=dev)
        wso = torch.empty(lrkv.project_workspace_bytes(nbt, DM, U * S * R), dtype=torch.uint8, device=dev)
        fns = [lambda a=a: lrkv.latent_project(x, a, 2 * U, R, h, wsl) for a in a_reps]
        rows[f"latent_project_kv_B{nbt}"] = _row(torch, fns, a_t.numel() * 2, 2 * nbt * a_t.numel())
        fns = [lambda w=w: lrkv.output_project(o, w, y, wso) for w in w_reps]
        rows[f"output_project_B{nbt}"] = _row(torch, fns, w_t.numel() * 2, 2 * nbt * w_t.numel())
    del a_t, w_t, a_reps, w_reps, x, o, h, y, wsl, wso, fns

    # chunked prefill on the RoPE path: Llama-2-7B layer, a 512-token chunk appended
    # at position 65024 attends causally over the 64K-token latent cache. Algorithmic
    # work: the reconstruction once per (token, head) plus scores and values per
    # (query, visible token); the kernel redoes the reconstruction per 128-query block
    # and forms scores from fp16 hi + lo parts (more MFMA work than counted)
    g.manual_seed(7)
    Tp, Mp = 65536, 512
    c = lrkv.LatentCache(1, U, S, GQ, DH, R, Tp, lrkv.FMT_FP16, THETA, device=dev)
    for t0 in range(0, Tp, 16384):
        c.append(torch.randn((1, U, 16384, R), generator=g, device=dev) * sq,
                 torch.randn((1, U, 16384, R), generator=g, device=dev) * sq)
    qp = torch.randn((1, Mp, U * S * GQ, DH), generator=g, device=dev)
    bkp = (torch.randn((U, R, S * DH), generator=g, device=dev) / 16).half()
    p0 = torch.full((1,), Tp - Mp, dtype=torch.int32, device=dev)
    reps = _latent_replicas(torch, lrkv, c, 2)
    wsp = [r.prefill_workspace(Mp) for r in reps]
    outp = torch.empty((1, Mp, U * S * GQ, R), dtype=torch.float32, device=dev)
    fns = [lambda r=r, w=w: r.prefill_attn(qp, bkp, p0, out=outp, workspace=w) for r, w in zip(reps, wsp)]
    heads = U * S * GQ
    vis = float(sum(Tp - Mp + m + 1 for m in range(Mp)))
    flops_p = 2.0 * R * DH * Tp * heads + 2.0 * (DH + R) * vis * heads
    row = _row(torch, fns, U * Tp * 2 * R * 2, flops_p, n=10)
    row["frac_mfma_peak"] = round(flops_p / (row["us_cold"] * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4)
    rows["prefill_chunk512_T65536"] = row
    del c, reps, qp, bkp, p0, wsp, outp, fns

    # RoPE path over Hadamard-rotated int4 latents: Llama-3-8B GQA, rank 64 per KV head
    g.manual_seed(4)
    B4, T4, H4, G4, R4 = 4, 65536, 8, 4, 64
    c = lrkv.LatentCache(B4, H4, 1, G4, DH, R4, T4, lrkv.FMT_INT4_G32, 5e5, device=dev)
    s4 = torch.exp(-torch.arange(R4, device=dev, dtype=torch.float32) / 64.0)
    for chunk in range(0, T4, 16384):
        hk = torch.randn((B4, H4, 16384, R4), generator=g, device=dev) * s4
        hv = torch.randn((B4, H4, 16384, R4), generator=g, device=dev) * s4
        c.append(hk, hv)
    del hk, hv
    q4 = torch.randn((B4, H4 * G4, DH), generator=g, device=dev)
    bk4 = (torch.randn((H4, R4, DH), generator=g, device=dev) / 8.0).half()
    out = torch.empty((B4, H4 * G4, R4), dtype=torch.float32, device=dev)
    reps = _latent_replicas(torch, lrkv, c, _n_replicas(_latent_bytes(c)))
    wss = [r.workspace(lrkv.MODE_ROPE_RECON) for r in reps]
    fns = [lambda r=r, w=w: lrkv.decode_attn(lrkv.MODE_ROPE_RECON, r.desc, q4, bk4, None, 0.0, out, w, T4)
           for r, w in zip(reps, wss)]
    rows["rope_int4_gqa_B4_T65536"] = _row(torch, fns, B4 * H4 * T4 * 72,
                                           B4 * H4 * T4 * (2 * R4 * DH + 2 * G4 * DH + 2 * G4 * R4),
                                           replica_bytes=_latent_bytes(c))
    # the whole step on the same caches: one token appended (int4, fused into the
    # query preparation) and decoded, one lrkv_decode_step call. Each call grows
    # its replica by one token; lengths start 256 below T4 (the tokens there are
    # overwritten) and stay within [T4 - 256, T4 - 256 + len_growth], so every
    # chunk keeps the decode row's 32 tiles
    nk4 = torch.randn((64, B4, H4, 1, R4), generator=g, device=dev) * s4
    nv4 = torch.randn((64, B4, H4, 1, R4), generator=g, device=dev) * s4
    for r in reps:
        r.host_lens[:] = T4 - 256
        r.lens.fill_(T4 - 256)
    wss = [r.workspace(lrkv.MODE_ROPE_RECON) for r in reps]   # valid up to length T4
    n_calls = [0]

    def step4(r, w):
        i = n_calls[0] % 64
        n_calls[0] += 1
        lrkv.decode_step(lrkv.MODE_ROPE_RECON, r.desc, nk4[i], nv4[i], 1, q4, bk4, None, 0.0, out, w, r.max_len)
        r.host_lens += 1

    fns = [lambda r=r, w=w: step4(r, w) for r, w in zip(reps, wss)]
    row = _row(torch, fns, B4 * H4 * T4 * 72, B4 * H4 * T4 * (2 * R4 * DH + 2 * G4 * DH + 2 * G4 * R4),
               replica_bytes=_latent_bytes(c))
    row["len_growth"] = int(max(r.max_len for r in reps)) - (T4 - 256)
    assert row["len_growth"] <= 256
    rows["rope_int4_gqa_step_B4_T65536"] = row
    del c, reps, q4, bk4, wss, out, fns, nk4, nv4

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
    out = torch.empty((B5, H5 * G5, DH), dtype=torch.float32, device=dev)
    n_dense, n_factored = 5, T5 // P5 - 5
    by = B5 * H5 * (n_factored * 2 * (P5 * RK + RK * DH) * 2 + n_dense * 2 * P5 * DH * 2)
    pbytes = lambda c: float(sum(t.numel() * t.element_size() for t in (c.dense_k, c.dense_v, c.lk, c.rk, c.lv, c.rv)))
    reps = _paged_replicas(torch, lrkv, pc, _n_replicas(pbytes(pc)))
    wss = [r.workspace() for r in reps]
    fns = [lambda r=r, w=w: r.decode(q5, out=out, workspace=w) for r, w in zip(reps, wss)]
    rows["hybrid_paged_B8_T32768"] = _row(torch, fns, by, replica_bytes=pbytes(pc))
    # one decode step's factorisation batch: one page per (b, head), keys and values
    step_pages = pages.view(B5, H5, -1, 3)[:, :, -1, :].reshape(-1, 3).contiguous()
    fct = _each_us(torch, [lambda: lrkv.factor_page(pc.desc, step_pages, step_pages.shape[0], k5, v5, T5, 0)], 20)
    rows["factor_pages_decode_batch"] = {"matrices": 2 * int(step_pages.shape[0]),
                                         "us_p10_p50_p90": _pct(fct)}
    rows["factor_pages_prefill_batch"] = {"matrices": 2 * n_fac, "us": round(prefill_ms * 1e3, 1)}
    del pc, reps, wss, fns

    # the same cache with int4 page factors (one fp16 scale per 32 stored elements):
    # codes + scales are (P r + r d) (1/2 + 2/32) bytes per factor pair
    pc4 = lrkv.PagedCache(B5, H5, G5, DH, P5, 1, 4, RK, RK, T5 // P5 + 8, device=dev,
                          factor_fmt=lrkv.FMT_INT4_G32)
    lrkv.factor_page(pc4.desc, pages, n_fac, k5, v5, T5, 0)
    lrkv.append_latent(lrkv.MODE_HYBRID_PAGED, pc4.desc, k5, v5, T5, 0)
    pc4.host_lens += T5
    torch.cuda.synchronize()
    per_side = (P5 * RK + RK * DH) // 2 + (P5 * RK + RK * DH) // 32 * 2
    by4 = B5 * H5 * (n_factored * 2 * per_side + n_dense * 2 * P5 * DH * 2)
    pbytes4 = lambda c: pbytes(c) + float(sum(t.numel() * t.element_size() for t in (c.lk_s, c.rk_s, c.lv_s, c.rv_s)))
    reps = _paged_replicas(torch, lrkv, pc4, _n_replicas(pbytes4(pc4)))
    wss = [r.workspace() for r in reps]
    fns = [lambda r=r, w=w: r.decode(q5, out=out, workspace=w) for r, w in zip(reps, wss)]
    rows["hybrid_paged_int4_B8_T32768"] = _row(torch, fns, by4, replica_bytes=pbytes4(pc4))
    del pc4, reps, wss, fns, k5, v5
    return rows


# ----------------------------------------------------------------------------- cpu baseline

def _cpu_info() -> dict:
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = None
    try:
        blas = np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {})
        blas = {k: blas.get(k) for k in ("name", "version", "openblas configuration") if k in blas}
    except Exception:  # pragma: no cover - older numpy
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "blas": blas}


def _median_time(fn, runs: int = 3, long_s: float = 2.0) -> float:
    """Median wall time of `runs` calls (one call when it alone takes over long_s)."""
    ts = []
    while len(ts) < runs:
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
        if ts[0] > long_s:
            break
    return float(np.median(ts))


def cpu_baseline() -> dict:
    """The float64 oracle timed on this host on bounded samples of each workload,
    at one thread and at all of the BLAS pool's threads: one unit (4 query heads)
    of the config-2 layer at T = 4K and 64K, one sequence-unit of the absorbed
    workload at 16K, one KV head (4 query heads) of the int4 grouped-query
    workload at 64K, one (sequence, KV head) of the hybrid workload at 32K, and the
    factorisation of one decode step's 128 page matrices; median of up to 3 runs."""
    import synth
    from oracle import attn as oattn
    from oracle import paged as opaged
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        all_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threadpool_limits = None
        all_threads = os.cpu_count() or 1

    samples = {}
    # config 2: one unit of the Llama-2-7B layer
    for T in (4096, 65536):
        lay = synth.latent_layer(2, 1, 1, T, R, S * DH, TAU)
        q = synth.queries(1002, 1, S * GQ, DH)
        hk, hv, Bk = oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"]), lay["Bk"].astype(np.float64)
        samples[f"rope_fp16_T{T}"] = (lambda hk=hk, hv=hv, Bk=Bk, q=q, T=T: oattn.palu_decode(
            hk, hv, Bk, q, [T], S, GQ, DH, THETA), T * BYTES_PER_UNIT_TOKEN, f"1 of 8 units (4 heads), T={T}")
        del lay
    # config 3: one sequence-unit of the absorbed workload
    lay = synth.latent_layer(3, 1, 1, 16384, R, S * DH, TAU)
    qa = synth.queries(1003, 1, S, R)
    hk3, hv3 = oattn.stored_fp16(lay["hk"]), oattn.stored_fp16(lay["hv"])
    samples["absorbed_fp16_T16384"] = (lambda: oattn.palu_decode_absorbed(hk3, hv3, qa, [16384], S, 1, DH),
                                       16384 * BYTES_PER_UNIT_TOKEN, "1 of 128 sequence-units (4 heads), T=16384")
    # config 4: one KV head of the int4 grouped-query workload
    lay = synth.latent_layer(4, 1, 1, 65536, 64, DH, 32.0)
    hk4, Bk4 = synth.hadamard_mixed(lay["hk"], lay["Bk"])
    hv4, _ = synth.hadamard_mixed(lay["hv"], lay["Bv"])
    hk4, hv4 = oattn.stored_int4(hk4), oattn.stored_int4(hv4)
    q4 = synth.queries(1004, 1, 4, DH)
    samples["rope_int4_gqa_T65536"] = (lambda: oattn.palu_decode(hk4, hv4, Bk4.astype(np.float64), q4, [65536],
                                                                 1, 4, DH, 5e5),
                                       65536 * 72, "1 of 32 (sequence, KV head) pairs (4 heads), T=65536")
    del lay
    # config 5: one (sequence, KV head) of the hybrid workload, and one decode step's factorisation batch
    T5, P5, RK = 32768, 32, 12
    dense = synth.paged_dense(5, 1, 1, T5, DH)
    fk = synth.factored_pages(6, T5 // P5, P5, DH, RK)
    fv = synth.factored_pages(7, T5 // P5, P5, DH, RK)
    Lk, Rk = (fk[n].astype(np.float64)[None, None] for n in ("L", "R"))
    Lv, Rv = (fv[n].astype(np.float64)[None, None] for n in ("L", "R"))
    q5 = synth.queries(1005, 1, 4, DH)
    by5 = ((T5 // P5 - 5) * 2 * (P5 * RK + RK * DH) * 2 + 5 * 2 * P5 * DH * 2)
    samples["hybrid_paged_T32768"] = (lambda: opaged.hybrid_decode(q5, [T5], dense["k"], dense["v"], Lk, Rk, Lv, Rv,
                                                                   P5, 1, 4, 4, form="reconstruct"),
                                      by5, "1 of 64 (sequence, KV head) pairs (4 heads), T=32768")
    pages = dense["k"][0, 0, :128 * P5].reshape(128, P5, DH).astype(np.float64)
    samples["factor_pages_decode_batch"] = (lambda: [opaged.factor_gram(pages[i], RK) for i in range(128)],
                                            0, "128 page matrices (32 x 128), Gram + eigh, rank 12")

    out = {}
    for threads in (1, all_threads):
        for name, (fn, nbytes, desc) in samples.items():
            if threadpool_limits is not None:
                with threadpool_limits(limits=threads):
                    t = _median_time(fn)
            else:
                t = _median_time(fn)
            ent = {"s": round(t, 4), "sample": desc}
            if nbytes:
                ent["GB_s"] = round(nbytes / t / 1e9, 4)
            out.setdefault(name, {})[f"threads_{threads}"] = ent
    head = out["rope_fp16_T65536"][f"threads_{all_threads}"]
    res = {"value": head["GB_s"], "unit": "GB/s", "cores": int(all_threads), "kind": "oracle",
           "sample": f"one unit (4 query heads) of the 8-unit Llama-2-7B layer at T=65536, float64 numpy oracle, "
                     f"median of up to 3 runs ({head['s']} s each), {all_threads} BLAS threads; the other "
                     f"workloads and one thread under configs"}
    res.update(_cpu_info())
    res["configs"] = out
    return res


# ----------------------------------------------------------------------------- power probe

def power_probe(torch, lrkv, c, w, q, Bk, n_split: int, launches: int = 2000) -> dict:
    """The partials kernel alone, `launches` back-to-back launches in one event pair
    after 200 untimed ones and a 0.5 s pause, on one cache: as generated, with every
    key latent zeroed, and with the queries zeroed (the same instruction stream and
    memory traffic, less switching in the multipliers). The cache and the prepared
    queries are restored afterwards."""
    mode, L = lrkv.MODE_ROPE_RECON, c.max_len

    def run() -> float:
        f = lambda: lrkv.decode_partials(mode, c.desc, None, 0.0, w, L, n_split)
        for _ in range(200):
            f()
        torch.cuda.synchronize()
        time.sleep(0.5)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(launches):
            f()
        b.record()
        torch.cuda.synchronize()
        return round(a.elapsed_time(b) / launches * 1e3, 2)

    prep = lambda qq: lrkv.decode_prepare(mode, c.desc, qq, Bk, None, 0.0, w, L, n_split)
    res = {"launches": launches}
    prep(q)
    res["us_random"] = run()
    hk = c.hk.clone()
    c.hk.zero_()
    res["us_keys_zero"] = run()
    c.hk.copy_(hk)
    del hk
    prep(torch.zeros_like(q))
    res["us_queries_zero"] = run()
    prep(q)
    res["us_random_again"] = run()
    torch.cuda.synchronize()
    return res


# ----------------------------------------------------------------------------- kernel-trace summary

def trace_summary(path: str, warmup: int, steps: int) -> dict:
    """Per-step statistics of the timed steps from a rocprofv3 kernel trace (CSV) of
    a bench run with the same warmup and steps. The main workload's steps come
    first: warmup + steps lrkv_decode_step steps (STEP_KERNELS in launch order),
    then the untimed pass of D steps issued as four calls (SPLIT_STEP_KERNELS),
    whose partials launches feed roofline.achieved."""
    import csv
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    names = set(SPLIT_STEP_KERNELS)

    def short(n):
        for k in names:
            if k in n:
                return k
        return None
    seq = [(short(r["Kernel_Name"]), int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rows]
    fused, split = [], []
    i = 0
    while i + 2 < len(seq):
        if i + 3 < len(seq) and tuple(x[0] for x in seq[i:i + 4]) == SPLIT_STEP_KERNELS:
            split.append(seq[i:i + 4])
            i += 4
        elif tuple(x[0] for x in seq[i:i + 3]) == STEP_KERNELS and not split:
            fused.append(seq[i:i + 3])
            i += 3
        else:
            i += 1
    timed = fused[warmup:warmup + steps]
    if len(timed) < steps:
        raise SystemExit(f"trace holds {len(fused)} decode steps, fewer than warmup + steps = {warmup + steps}")
    out = {"steps_in_trace": len(fused), "timed_steps": len(timed)}
    for j, k in enumerate(STEP_KERNELS):
        d = np.array([(x[j][2] - x[j][1]) / 1e3 for x in timed])
        out[k + "_us"] = {"mean": round(float(d.mean()), 2), "p10_p50_p90": _pct(d)}
    whole = np.array([(x[-1][2] - x[0][1]) / 1e3 for x in timed])
    period = np.diff([x[0][1] for x in timed] + [timed[-1][-1][2]]) / 1e3
    out["step_us"] = {"mean": round(float(whole.mean()), 2), "p10_p50_p90": _pct(whole)}
    out["step_period_us"] = {"mean": round(float(period.mean()), 2), "p10_p50_p90": _pct(period)}
    # the untimed pass right after the timed steps (the same D as in main())
    D = max(20, min(steps, 200))
    if len(split) >= D:
        d = np.array([(x[2][2] - x[2][1]) / 1e3 for x in split[:D]])
        out["partials_us_roofline_pass"] = {"launches": D, "mean": round(float(d.mean()), 2),
                                            "p10_p50_p90": _pct(d)}
    return out


# ----------------------------------------------------------------------------- main

def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--T", type=int, default=65536)
    ap.add_argument("--replicas", type=int, default=2)
    ap.add_argument("--n-split", type=int, default=0)
    ap.add_argument("--sustained", type=int, default=2000,
                    help="steps of the untimed sustained pass reported under detail (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--power-probe", action="store_true",
                    help="also time the partials kernel sustained on the benchmark cache, with its "
                         "keys zeroed, and with the queries zeroed (how much the kernel's speed "
                         "depends on the data it multiplies; detail.power_probe)")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the timing of the other hot-path rows (absorbed, int4, hybrid, factorisation)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a 1 GiB device copy (reference for HBM counter scaling)")
    ap.add_argument("--trace-summary", metavar="CSV",
                    help="summarise the timed steps of a rocprofv3 kernel trace of a bench run and exit")
    args = ap.parse_args()

    if args.trace_summary:
        print(json.dumps(trace_summary(args.trace_summary, args.warmup, args.steps)))
        return 0

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
    T, K, W, NR = args.T, args.steps, args.warmup, max(1, args.replicas)
    D = max(20, min(K, 200))              # untimed pass with events around each step's partials kernel
    n5 = 8                                # untimed steps with every phase bracketed
    SU = max(0, args.sustained)
    n_tok = W + K + D + n5 + SU
    # lengths start so that the timed steps' mean length is T
    T_init = T - 1 - (W + K // 2) // NR
    cap = ((T_init + n_tok // NR + NR + 64) // 32 + 1) * 32

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
    step_tok = synth.latent_layer(3, B, U, 64, R, S * DH, TAU)
    nk = torch.from_numpy(step_tok["hk"]).to(dev)
    nv = torch.from_numpy(step_tok["hv"]).to(dev)
    new_k = [nk[:, :, i:i + 1].contiguous() for i in range(64)]
    new_v = [nv[:, :, i:i + 1].contiguous() for i in range(64)]
    q = torch.from_numpy(synth.queries(1002, B, U * S * GQ, DH)).to(dev)
    out = torch.empty((B, U * S * GQ, R), dtype=torch.float32, device=dev)
    for c in reps:          # the workspace must cover the longest length of the run
        c.host_lens += n_tok // NR + 1
    ws = [c.workspace(lrkv.MODE_ROPE_RECON, args.n_split) for c in reps]
    for c in reps:
        c.host_lens -= n_tok // NR + 1
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
        """One decode step on replica i % NR: one lrkv_decode_step call, or with ev the
        same work as four calls with two events recorded around its partials kernel,
        or five around every phase."""
        c, w = reps[i % NR], ws[i % NR]
        if ev is None:
            L0 = c.max_len
            lrkv.decode_step(mode, c.desc, new_k[i % 64], new_v[i % 64], 1, q, Bk, None, 0.0, out, w, L0,
                             args.n_split, stream=stream)
            c.host_lens += 1
            return L0 + 1
        five = len(ev) == 5
        if five:
            ev[0].record()
        c.append(new_k[i % 64], new_v[i % 64], stream=stream)
        L = c.max_len
        if five:
            ev[1].record()
        lrkv.decode_prepare(mode, c.desc, q, Bk, None, 0.0, w, L, args.n_split, stream=stream)
        if ev is not None:
            ev[2 if five else 0].record()
        lrkv.decode_partials(mode, c.desc, None, 0.0, w, L, args.n_split, stream=stream)
        if ev is not None:
            ev[3 if five else 1].record()
        lrkv.merge_partials(mode, c.desc, out, w, L, args.n_split, stream=stream)
        if five:
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
    # untimed pass right after: whole steps issued as in the timed region, with two
    # events around each partials kernel (the kernel's in-step duration), then a few
    # steps with every phase bracketed
    pev = [mk(2) for _ in range(D)]
    lens_d = [step(W + K + k, pev[k]) for k in range(D)]
    torch.cuda.synchronize()
    part_each = np.array([a.elapsed_time(b) for a, b in pev])
    dev_ev = [mk(5) for _ in range(n5)]
    for k in range(n5):
        step(W + K + D + k, dev_ev[k])
    torch.cuda.synchronize()
    ph = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in dev_ev])
    # sustained pass: SU more steps in one event pair (the power-limited steady state)
    sustained = None
    if SU:
        s0, s1 = mk(2)
        s0.record()
        lens_su = [step(W + K + D + n5 + k) for k in range(SU)]
        s1.record()
        torch.cuda.synchronize()
        su_ms = s0.elapsed_time(s1)
        su_bytes = U * B * np.array(lens_su, np.float64) * BYTES_PER_UNIT_TOKEN
        sustained = {"steps": SU, "us_per_step": round(su_ms / SU * 1e3, 2),
                     "GB_s": round(su_bytes.sum() / (su_ms * 1e-3) / 1e9, 1)}

    lens_timed = np.array(lens_timed, dtype=np.float64)
    bytes_steps = U * B * lens_timed * BYTES_PER_UNIT_TOKEN
    flops_steps = U * B * lens_timed * FLOP_PER_UNIT_TOKEN
    gbs = bytes_steps.sum() / (total_ms * 1e-3) / 1e9
    part_ms = float(part_each.mean())
    achieved = U * B * float(np.mean(lens_d)) * BYTES_PER_UNIT_TOKEN / (part_ms * 1e-3) / 1e9
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
            "kernel": "rope_decode_fw (lrkv_decode_partials)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "detail": {
            "partials_us_in_step_mean_p10_p50_p90": [round(part_ms * 1e3, 2)] + _pct(part_each * 1e3),
            "partials_in_step_steps": D,
            "phase_us_untimed_pass": {"append": round(ph[:, 0].mean() * 1e3, 2),
                                      "prepare": round(ph[:, 1].mean() * 1e3, 2),
                                      "partials": round(ph[:, 2].mean() * 1e3, 2),
                                      "merge": round(ph[:, 3].mean() * 1e3, 2)},
            "sustained": sustained,
            "mfma_tflops_partials": round(flops_steps.mean() / (part_ms * 1e-3) / 1e12, 1),
            "mfma_frac_partials": round(flops_steps.mean() / (part_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
            "bytes_per_step": float(bytes_steps.mean()),
            "host_submit_us_per_step": round(host_us, 1),
            "output_finite": ok,
        },
    }
    if args.power_probe:
        log("bench: power probe (partials sustained on random / zeroed operands)")
        result["detail"]["power_probe"] = power_probe(torch, lrkv, reps[0], ws[0], q, Bk, args.n_split)
    del reps, ws
    torch.cuda.empty_cache()
    log("bench: streaming-read reference")
    sr = measure_stream_read(torch, lrkv, dev)
    result["detail"]["stream_read"] = sr
    result["detail"]["partials_frac_stream_read"] = round(achieved / sr["GB_s"], 4)
    if not args.no_rows:
        log("bench: timing the other hot-path rows (cold and warm cache)")
        rows = measure_rows(torch, lrkv, dev)
        for r in rows.values():
            if "GB_s" in r:
                r["frac_stream_read"] = round(r["GB_s"] / sr["GB_s"], 4)
        result["detail"]["rows"] = rows
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on the host (cpu_baseline)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)
    return 0 if ok else 1


if __name__ == "__main__":
    sys.exit(main())
