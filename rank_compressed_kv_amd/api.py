"""Python binding of liblrkv.so with the C entry points' names.

Argument marshalling only: tensors are passed as device pointers together with
the current HIP stream; every step of the decode path runs in the library's
kernels. PyTorch is used to allocate device memory (the caches, outputs and
workspaces) and to supply streams.
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _lib as L
from ._lib import (BLOCK, FMT_FP16, FMT_INT4_G32, MODE_ABSORBED, MODE_HYBRID_PAGED,
                   MODE_ROPE_RECON, PAGE_EMPTY, LatentCacheDesc, PagedCacheDesc, LrkvError)

__all__ = [
    "decode_workspace_bytes", "append_latent", "decode_attn", "decode_attn_noalloc", "decode_step",
    "decode_prepare",
    "decode_partials",
    "merge_partials", "factor_page", "paged_plan", "project_workspace_bytes", "latent_project",
    "output_project", "probe_stream_read",
    "LatentCache", "PagedCache", "LrkvError",
    "MODE_ROPE_RECON", "MODE_ABSORBED", "MODE_HYBRID_PAGED", "FMT_FP16", "FMT_INT4_G32",
]


def _p(t) -> ctypes.c_void_p | None:
    """Raw pointer of a tensor handed to the C ABI, which reads dense row-major memory."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError(f"tensor of shape {tuple(t.shape)} is not contiguous (the C ABI reads row-major memory)")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, dtype, shape, name: str):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: expected contiguous device {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


# ----------------------------------------------------------------------------- C entry points

def decode_workspace_bytes(mode: int, desc, host_max_len: int, n_split: int = 0) -> int:
    return int(L.lib().lrkv_decode_workspace_bytes(mode, ctypes.byref(desc), host_max_len, n_split))


def append_latent(mode: int, desc, new_k, new_v, n_new: int, host_max_len: int, stream=None) -> None:
    L.check(L.lib().lrkv_append_latent(mode, ctypes.byref(desc), _p(new_k), _p(new_v), n_new,
                                       host_max_len, _stream(stream)), "lrkv_append_latent")


def decode_attn(mode: int, desc, q, bk, q_pos, sm_scale: float, out, workspace,
                host_max_len: int, n_split: int = 0, stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    L.check(L.lib().lrkv_decode_attn(mode, ctypes.byref(desc), _p(q), _p(bk), _p(q_pos),
                                     float(sm_scale), _p(out), _p(workspace), ws_bytes,
                                     host_max_len, n_split, _stream(stream)), "lrkv_decode_attn")


def decode_step(mode: int, desc, new_k, new_v, n_new: int, q, bk, q_pos, sm_scale: float, out, workspace,
                host_max_len: int, n_split: int = 0, stream=None) -> None:
    """Append n_new tokens, then decode (lrkv_decode_step): host_max_len bounds the
    lengths before the append, the workspace covers host_max_len + n_new."""
    L.check(L.lib().lrkv_decode_step(mode, ctypes.byref(desc), _p(new_k), _p(new_v), n_new, _p(q), _p(bk),
                                      _p(q_pos), float(sm_scale), _p(out), _p(workspace), _ws(workspace),
                                      host_max_len, n_split, _stream(stream)), "lrkv_decode_step")


def decode_attn_noalloc(mode: int, desc, q, bk, q_pos, sm_scale: float, out, host_max_len: int,
                        n_split: int = 0, stream=None) -> None:
    """lrkv_decode_attn with the library's static device scratch as its workspace."""
    L.check(L.lib().lrkv_decode_attn_noalloc(mode, ctypes.byref(desc), _p(q), _p(bk), _p(q_pos),
                                             float(sm_scale), _p(out), host_max_len, n_split,
                                             _stream(stream)), "lrkv_decode_attn_noalloc")


def _ws(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def decode_prepare(mode: int, desc, q, bk, q_pos, sm_scale: float, workspace, host_max_len: int,
                   n_split: int = 0, stream=None) -> None:
    L.check(L.lib().lrkv_decode_prepare(mode, ctypes.byref(desc), _p(q), _p(bk), _p(q_pos),
                                        float(sm_scale), _p(workspace), _ws(workspace), host_max_len,
                                        n_split, _stream(stream)), "lrkv_decode_prepare")


def decode_partials(mode: int, desc, q, sm_scale: float, workspace, host_max_len: int,
                    n_split: int = 0, stream=None) -> None:
    L.check(L.lib().lrkv_decode_partials(mode, ctypes.byref(desc), _p(q), float(sm_scale),
                                         _p(workspace), _ws(workspace), host_max_len, n_split,
                                         _stream(stream)), "lrkv_decode_partials")


def merge_partials(mode: int, desc, out, workspace, host_max_len: int, n_split: int = 0,
                   stream=None) -> None:
    L.check(L.lib().lrkv_merge_partials(mode, ctypes.byref(desc), _p(out), _p(workspace),
                                        _ws(workspace), host_max_len, n_split, _stream(stream)),
            "lrkv_merge_partials")


def factor_page(desc, pages, n_pages: int, src_k=None, src_v=None, src_len: int = 0,
                max_sweeps: int = 0, stream=None) -> None:
    L.check(L.lib().lrkv_factor_page(ctypes.byref(desc), _p(pages), n_pages, _p(src_k), _p(src_v),
                                     src_len, max_sweeps, _stream(stream)), "lrkv_factor_page")


def project_workspace_bytes(m: int, n: int, k: int) -> int:
    return int(L.lib().lrkv_project_workspace_bytes(m, n, k))


def _proj_ws(m, n, k, workspace, device):
    need = project_workspace_bytes(m, n, k)
    if need == 0:
        raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_project_workspace_bytes")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace


def latent_project(x, a_t, units: int, rank: int, h=None, workspace=None, stream=None):
    """h = x A for every unit: x float32 [n_tok][d_model], a_t float16
    [units * rank][d_model] -> h float32 [n_tok][units][rank]."""
    n_tok, d_model = x.shape
    _need(x, torch.float32, (n_tok, d_model), "x")
    _need(a_t, torch.float16, (units * rank, d_model), "a_t")
    if h is None:
        h = torch.empty((n_tok, units, rank), dtype=torch.float32, device=x.device)
    _need(h, torch.float32, (n_tok, units, rank), "h")
    workspace = _proj_ws(n_tok, units * rank, d_model, workspace, x.device)
    L.check(L.lib().lrkv_latent_project(_p(x), n_tok, d_model, _p(a_t), units, rank, _p(h), _p(workspace),
                                        _ws(workspace), _stream(stream)), "lrkv_latent_project")
    return h


def output_project(o, w_t, y=None, workspace=None, stream=None):
    """y = sum_j o_j (B^v_j W^o_j): o float32 [batch][q_heads][rank], w_t float16
    [d_model][q_heads * rank] -> y float32 [batch][d_model]."""
    batch, q_heads, rank = o.shape
    d_model = w_t.shape[0]
    _need(o, torch.float32, (batch, q_heads, rank), "o")
    _need(w_t, torch.float16, (d_model, q_heads * rank), "w_t")
    if y is None:
        y = torch.empty((batch, d_model), dtype=torch.float32, device=o.device)
    _need(y, torch.float32, (batch, d_model), "y")
    workspace = _proj_ws(batch, d_model, q_heads * rank, workspace, o.device)
    L.check(L.lib().lrkv_output_project(_p(o), batch, q_heads, rank, _p(w_t), d_model, _p(y), _p(workspace),
                                        _ws(workspace), _stream(stream)), "lrkv_output_project")
    return y


def probe_stream_read(buf, out, blocks: int = 4096, stream=None) -> None:
    """Measurement aid: one streaming read of every byte of device tensor `buf`
    (out: device uint8/int32 tensor of at least 4 * blocks bytes)."""
    nbytes = buf.numel() * buf.element_size()
    L.check(L.lib().lrkv_probe_stream_read(_p(buf), nbytes, _p(out), blocks, _stream(stream)),
            "lrkv_probe_stream_read")


def paged_plan(desc, host_lens: np.ndarray, n_new: int) -> np.ndarray:
    lens = np.ascontiguousarray(host_lens, dtype=np.int32)
    n = L.check(L.lib().lrkv_paged_plan(ctypes.byref(desc), lens.ctypes.data, n_new, None, 0),
                "lrkv_paged_plan")
    out = np.zeros((max(n, 1), 3), dtype=np.int32)
    if n:
        L.check(L.lib().lrkv_paged_plan(ctypes.byref(desc), lens.ctypes.data, n_new,
                                        out.ctypes.data, n), "lrkv_paged_plan")
    return out[:n]


# ----------------------------------------------------------------------------- cache objects

class LatentCache:
    """Device buffers of a Palu latent cache (layouts in include/lrkv.h) plus the host
    mirror of the sequence lengths."""

    def __init__(self, batch: int, units: int, kv_per_unit: int, q_per_kv: int, head_dim: int,
                 rank: int, capacity: int, fmt: int = FMT_FP16, rope_theta: float = 0.0,
                 device="cuda"):
        if capacity % BLOCK:
            raise ValueError("capacity must be a multiple of 32")
        self.B, self.U, self.s, self.gq, self.dh, self.r = batch, units, kv_per_unit, q_per_kv, head_dim, rank
        self.cap, self.fmt, self.theta = capacity, fmt, float(rope_theta)
        self.Hq = units * kv_per_unit * q_per_kv
        dev = torch.device(device)
        if fmt == FMT_FP16:
            self.hk = torch.zeros((batch, units, capacity, rank), dtype=torch.float16, device=dev)
            self.hv = torch.zeros((batch, units, capacity // BLOCK, rank, BLOCK), dtype=torch.float16, device=dev)
            self.sk = self.sv = None
        elif fmt == FMT_INT4_G32:
            self.hk = torch.zeros((batch, units, capacity, rank // 2), dtype=torch.uint8, device=dev)
            self.sk = torch.zeros((batch, units, capacity, rank // 32), dtype=torch.float16, device=dev)
            self.hv = torch.zeros((batch, units, capacity // BLOCK, rank, BLOCK // 2), dtype=torch.uint8, device=dev)
            self.sv = torch.zeros((batch, units, capacity // BLOCK, rank // 32, BLOCK), dtype=torch.float16, device=dev)
        else:
            raise ValueError("fmt must be FMT_FP16 or FMT_INT4_G32")
        self.lens = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.host_lens = np.zeros(batch, dtype=np.int64)
        self.desc = LatentCacheDesc(batch, units, kv_per_unit, q_per_kv, head_dim, rank, capacity, fmt,
                                    self.theta, self.hk.data_ptr(), self.hv.data_ptr(),
                                    0 if self.sk is None else self.sk.data_ptr(),
                                    0 if self.sv is None else self.sv.data_ptr(), self.lens.data_ptr())

    @property
    def max_len(self) -> int:
        return int(self.host_lens.max())

    def reset(self) -> None:
        self.lens.zero_()
        self.host_lens[:] = 0

    def append(self, new_k: torch.Tensor, new_v: torch.Tensor, stream=None) -> None:
        """new_k, new_v: device float32 [B][U][n_new][r]."""
        n_new = new_k.shape[2]
        _need(new_k, torch.float32, (self.B, self.U, n_new, self.r), "new_k")
        _need(new_v, torch.float32, (self.B, self.U, n_new, self.r), "new_v")
        append_latent(MODE_ROPE_RECON, self.desc, new_k, new_v, n_new, self.max_len, stream)
        self.host_lens += n_new

    def workspace(self, mode: int, n_split: int = 0) -> torch.Tensor:
        n = decode_workspace_bytes(mode, self.desc, self.max_len, n_split)
        if n == 0:
            raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_decode_workspace_bytes")
        return torch.empty(n, dtype=torch.uint8, device=self.hk.device)

    def decode(self, mode: int, q: torch.Tensor, bk: torch.Tensor | None = None,
               q_pos: torch.Tensor | None = None, sm_scale: float = 0.0, n_split: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        """ROPE_RECON: q float32 [B][Hq][d_h], bk float16 [U][r][s*d_h].
        ABSORBED: q float32 [B][Hq][r]. Returns float32 [B][Hq][r]."""
        qdim = self.dh if mode == MODE_ROPE_RECON else self.r
        _need(q, torch.float32, (self.B, self.Hq, qdim), "q")
        if bk is not None:
            _need(bk, torch.float16, (self.U, self.r, self.s * self.dh), "bk")
        if q_pos is not None:
            _need(q_pos, torch.int32, (self.B,), "q_pos")
        if out is None:
            out = torch.empty((self.B, self.Hq, self.r), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(mode, n_split)
        decode_attn(mode, self.desc, q, bk, q_pos, sm_scale, out, workspace, self.max_len, n_split, stream)
        return out

    def step(self, mode: int, new_k: torch.Tensor, new_v: torch.Tensor, q: torch.Tensor,
             bk: torch.Tensor | None = None, q_pos: torch.Tensor | None = None, sm_scale: float = 0.0,
             n_split: int = 0, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             stream=None) -> torch.Tensor:
        """append(new_k, new_v) then decode(mode, q, ...) in one call (lrkv_decode_step);
        the workspace must cover the lengths after the append."""
        n_new = new_k.shape[2]
        _need(new_k, torch.float32, (self.B, self.U, n_new, self.r), "new_k")
        _need(new_v, torch.float32, (self.B, self.U, n_new, self.r), "new_v")
        qdim = self.dh if mode == MODE_ROPE_RECON else self.r
        _need(q, torch.float32, (self.B, self.Hq, qdim), "q")
        if bk is not None:
            _need(bk, torch.float16, (self.U, self.r, self.s * self.dh), "bk")
        if q_pos is not None:
            _need(q_pos, torch.int32, (self.B,), "q_pos")
        if out is None:
            out = torch.empty((self.B, self.Hq, self.r), dtype=torch.float32, device=q.device)
        if workspace is None:
            n = decode_workspace_bytes(mode, self.desc, self.max_len + n_new, n_split)
            if n == 0:
                raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_decode_workspace_bytes")
            workspace = torch.empty(n, dtype=torch.uint8, device=self.hk.device)
        decode_step(mode, self.desc, new_k, new_v, n_new, q, bk, q_pos, sm_scale, out, workspace, self.max_len,
                    n_split, stream)
        self.host_lens += n_new
        return out

    def prefill_workspace(self, m_tokens: int) -> torch.Tensor:
        n = int(L.lib().lrkv_prefill_workspace_bytes(ctypes.byref(self.desc), m_tokens, self.max_len))
        if n == 0:
            raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_prefill_workspace_bytes")
        return torch.empty(n, dtype=torch.uint8, device=self.hk.device)

    def prefill_attn(self, q: torch.Tensor, bk: torch.Tensor, p0: torch.Tensor, sm_scale: float = 0.0,
                     out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
        """Causal attention of a chunk of m new tokens (already appended at positions
        p0[b] .. p0[b] + m - 1): q float32 [B][m][Hq][d_h], bk float16 [U][r][s*d_h],
        p0 int32 [B] -> float32 [B][m][Hq][r]."""
        m = q.shape[1]
        _need(q, torch.float32, (self.B, m, self.Hq, self.dh), "q")
        _need(bk, torch.float16, (self.U, self.r, self.s * self.dh), "bk")
        _need(p0, torch.int32, (self.B,), "p0")
        if out is None:
            out = torch.empty((self.B, m, self.Hq, self.r), dtype=torch.float32, device=q.device)
        _need(out, torch.float32, (self.B, m, self.Hq, self.r), "out")
        if workspace is None:
            workspace = self.prefill_workspace(m)
        L.check(L.lib().lrkv_prefill_attn(ctypes.byref(self.desc), _p(q), _p(bk), _p(p0), m, self.max_len,
                                          float(sm_scale), _p(out), _p(workspace), _ws(workspace),
                                          _stream(stream)), "lrkv_prefill_attn")
        return out


class PagedCache:
    """Device buffers of a PuzzleKV-style hybrid cache (layouts in include/lrkv.h)."""

    def __init__(self, batch: int, kv_heads: int, q_per_kv: int, head_dim: int = 128,
                 page_size: int = 32, sink_pages: int = 1, window_pages: int = 4, rank_k: int = 12,
                 rank_v: int = 12, max_pages: int = 1024, device="cuda", factor_fmt: int = FMT_FP16):
        self.B, self.H, self.G, self.d, self.P = batch, kv_heads, q_per_kv, head_dim, page_size
        self.sink, self.window, self.rk_, self.rv_, self.max_pages = sink_pages, window_pages, rank_k, rank_v, max_pages
        dev = torch.device(device)
        nd = sink_pages + window_pages
        f16 = torch.float16
        # keys row-major; values (dense and factored) dimension-major
        self.dense_k = torch.zeros((batch, kv_heads, nd, page_size, head_dim), dtype=f16, device=dev)
        self.dense_v = torch.zeros((batch, kv_heads, nd, head_dim, page_size), dtype=f16, device=dev)
        self.factor_fmt = factor_fmt
        if factor_fmt == FMT_FP16:
            self.lk = torch.zeros((batch, kv_heads, max_pages, page_size, rank_k), dtype=f16, device=dev)
            self.rk = torch.zeros((batch, kv_heads, max_pages, rank_k, head_dim), dtype=f16, device=dev)
            self.lv = torch.zeros((batch, kv_heads, max_pages, rank_v, page_size), dtype=f16, device=dev)
            self.rv = torch.zeros((batch, kv_heads, max_pages, head_dim, rank_v), dtype=f16, device=dev)
            self.lk_s = self.rk_s = self.lv_s = self.rv_s = None
        elif factor_fmt == FMT_INT4_G32:
            # codes, two per byte, in the fp16 layouts' element order; one fp16 scale
            # per 32 consecutive elements of a page's factor
            u8 = torch.uint8
            nl_k, nr_k = page_size * rank_k, rank_k * head_dim
            nl_v, nr_v = page_size * rank_v, rank_v * head_dim
            shp = (batch, kv_heads, max_pages)
            self.lk = torch.zeros(shp + (nl_k // 2,), dtype=u8, device=dev)
            self.rk = torch.zeros(shp + (nr_k // 2,), dtype=u8, device=dev)
            self.lv = torch.zeros(shp + (nl_v // 2,), dtype=u8, device=dev)
            self.rv = torch.zeros(shp + (nr_v // 2,), dtype=u8, device=dev)
            self.lk_s = torch.zeros(shp + (nl_k // 32,), dtype=f16, device=dev)
            self.rk_s = torch.zeros(shp + (nr_k // 32,), dtype=f16, device=dev)
            self.lv_s = torch.zeros(shp + (nl_v // 32,), dtype=f16, device=dev)
            self.rv_s = torch.zeros(shp + (nr_v // 32,), dtype=f16, device=dev)
        else:
            raise ValueError("factor_fmt must be FMT_FP16 or FMT_INT4_G32")
        self.page_table = torch.full((batch, kv_heads, max_pages), PAGE_EMPTY, dtype=torch.int32, device=dev)
        self.lens = torch.zeros(batch, dtype=torch.int32, device=dev)
        self.host_lens = np.zeros(batch, dtype=np.int64)
        self.desc = PagedCacheDesc(batch, kv_heads, q_per_kv, head_dim, page_size, sink_pages, window_pages,
                                   rank_k, rank_v, max_pages, self.dense_k.data_ptr(), self.dense_v.data_ptr(),
                                   self.lk.data_ptr(), self.rk.data_ptr(), self.lv.data_ptr(),
                                   self.rv.data_ptr(), self.page_table.data_ptr(), self.lens.data_ptr(),
                                   factor_fmt, *(0 if t is None else t.data_ptr()
                                                 for t in (self.lk_s, self.rk_s, self.lv_s, self.rv_s)))

    @property
    def max_len(self) -> int:
        return int(self.host_lens.max())

    def reset(self) -> None:
        self.page_table.fill_(PAGE_EMPTY)
        self.lens.zero_()
        self.host_lens[:] = 0

    def _pages(self, n_new: int) -> torch.Tensor | None:
        plan = paged_plan(self.desc, self.host_lens, n_new)
        if len(plan) == 0:
            return None
        return torch.from_numpy(plan).to(self.dense_k.device)

    def prefill(self, k: torch.Tensor, v: torch.Tensor, max_sweeps: int = 0, stream=None) -> None:
        """k, v: device float16 [B][H][T][d] for fresh sequences: factors every page that
        leaves the window directly from k/v, then appends all tokens."""
        if self.max_len != 0:
            raise ValueError("prefill needs empty sequences")
        T = k.shape[2]
        _need(k, torch.float16, (self.B, self.H, T, self.d), "k")
        _need(v, torch.float16, (self.B, self.H, T, self.d), "v")
        pages = self._pages(T)
        if pages is not None:
            factor_page(self.desc, pages, pages.shape[0], k, v, T, max_sweeps, stream)
        append_latent(MODE_HYBRID_PAGED, self.desc, k, v, T, 0, stream)
        self.host_lens += T

    def append(self, k: torch.Tensor, v: torch.Tensor, max_sweeps: int = 0, stream=None) -> None:
        """One decode token per sequence, k, v device float16 [B][H][1][d]: the page that
        leaves the window (if any) is factored from its dense slot first."""
        _need(k, torch.float16, (self.B, self.H, 1, self.d), "k")
        _need(v, torch.float16, (self.B, self.H, 1, self.d), "v")
        pages = self._pages(1)
        if pages is not None:
            factor_page(self.desc, pages, pages.shape[0], None, None, 0, max_sweeps, stream)
        append_latent(MODE_HYBRID_PAGED, self.desc, k, v, 1, self.max_len, stream)
        self.host_lens += 1

    def step(self, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, sm_scale: float = 0.0,
             n_split: int = 0, out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
             max_sweeps: int = 0, stream=None) -> torch.Tensor:
        """append(k, v) then decode(q) (lrkv_decode_step): the page that leaves the
        window (if any) is factored first, as append does; the workspace must cover
        the lengths after the append."""
        _need(k, torch.float16, (self.B, self.H, 1, self.d), "k")
        _need(v, torch.float16, (self.B, self.H, 1, self.d), "v")
        _need(q, torch.float32, (self.B, self.H * self.G, self.d), "q")
        pages = self._pages(1)
        if pages is not None:
            factor_page(self.desc, pages, pages.shape[0], None, None, 0, max_sweeps, stream)
        if out is None:
            out = torch.empty((self.B, self.H * self.G, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            n = decode_workspace_bytes(MODE_HYBRID_PAGED, self.desc, self.max_len + 1, n_split)
            if n == 0:
                raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_decode_workspace_bytes")
            workspace = torch.empty(n, dtype=torch.uint8, device=self.dense_k.device)
        decode_step(MODE_HYBRID_PAGED, self.desc, k, v, 1, q, None, None, sm_scale, out, workspace,
                    self.max_len, n_split, stream)
        self.host_lens += 1
        return out

    def workspace(self, n_split: int = 0) -> torch.Tensor:
        n = decode_workspace_bytes(MODE_HYBRID_PAGED, self.desc, self.max_len, n_split)
        if n == 0:
            raise LrkvError(L.LRKV_ERR_INVALID_ARG, "lrkv_decode_workspace_bytes")
        return torch.empty(n, dtype=torch.uint8, device=self.dense_k.device)

    def decode(self, q: torch.Tensor, sm_scale: float = 0.0, n_split: int = 0,
               out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
               stream=None) -> torch.Tensor:
        """q float32 [B][H*G][d] -> float32 [B][H*G][d]."""
        _need(q, torch.float32, (self.B, self.H * self.G, self.d), "q")
        if out is None:
            out = torch.empty((self.B, self.H * self.G, self.d), dtype=torch.float32, device=q.device)
        if workspace is None:
            workspace = self.workspace(n_split)
        decode_attn(MODE_HYBRID_PAGED, self.desc, q, None, None, sm_scale, out, workspace,
                    self.max_len, n_split, stream)
        return out
