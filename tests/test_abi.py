"""The C ABI without a GPU: exported symbols, host-side validation, the paged planner.

No call here reaches a kernel launch: every call either fails validation on the
host or is host-only (lrkv_paged_plan, lrkv_decode_workspace_bytes)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import paged as opaged
from rank_compressed_kv_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000          # non-null, 16-byte aligned, never dereferenced by host code


@pytest.fixture(scope="module")
def lib():
    return L.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "lrkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrkv_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert set(names) == set(L.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert L.status_string(code) and L.status_string(code) != "unknown status"
    assert lib.lrkv_version() >= 100


def _latent(**kw):
    f = dict(batch=1, units=8, kv_per_unit=4, q_per_kv=1, head_dim=128, rank=256, capacity=4096,
             fmt=0, rope_theta=1e4, hk=FAKE, hv=FAKE, sk=0, sv=0, lens=FAKE)
    f.update(kw)
    return L.LatentCacheDesc(*[f[n] for n, _ in L.LatentCacheDesc._fields_])


def _paged(**kw):
    f = dict(batch=2, kv_heads=2, q_per_kv=4, head_dim=128, page_size=32, sink_pages=1, window_pages=4,
             rank_k=12, rank_v=12, max_pages=64, dense_k=FAKE, dense_v=FAKE, lk=FAKE, rk=FAKE, lv=FAKE,
             rv=FAKE, page_table=FAKE, lens=FAKE, factor_fmt=0, lk_s=None, rk_s=None, lv_s=None, rv_s=None)
    f.update(kw)
    return L.PagedCacheDesc(*[f[n] for n, _ in L.PagedCacheDesc._fields_])


def test_append_validation(lib):
    d = _latent()
    ok = ctypes.c_void_p(FAKE)
    assert lib.lrkv_append_latent(0, None, ok, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_append_latent(0, ctypes.byref(d), None, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_append_latent(0, ctypes.byref(d), ok, ok, 0, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_append_latent(0, ctypes.byref(d), ok, ok, 1, 4096, None) == L.LRKV_ERR_CAPACITY
    assert lib.lrkv_append_latent(0, ctypes.byref(d), ok, ok, 4097, 0, None) == L.LRKV_ERR_CAPACITY
    assert lib.lrkv_append_latent(7, ctypes.byref(d), ok, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG
    bad = _latent(capacity=100)
    assert lib.lrkv_append_latent(0, ctypes.byref(bad), ok, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG
    i4 = _latent(fmt=1, rank=48, sk=FAKE, sv=FAKE)
    assert lib.lrkv_append_latent(0, ctypes.byref(i4), ok, ok, 1, 0, None) == L.LRKV_ERR_UNSUPPORTED
    i4n = _latent(fmt=1, rank=64)
    assert lib.lrkv_append_latent(0, ctypes.byref(i4n), ok, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG
    unal = ctypes.c_void_p(FAKE + 4)
    assert lib.lrkv_append_latent(0, ctypes.byref(d), unal, ok, 1, 0, None) == L.LRKV_ERR_INVALID_ARG


def test_decode_validation(lib):
    d = _latent()
    ok = ctypes.c_void_p(FAKE)
    need = lib.lrkv_decode_workspace_bytes(0, ctypes.byref(d), 4096, 0)
    assert need > 0
    assert lib.lrkv_decode_workspace_bytes(0, ctypes.byref(d), 4097, 0) == 0
    call = lambda mode, bk, qpos, ws, nbytes, T=4096, desc=d: lib.lrkv_decode_attn(
        mode, ctypes.byref(desc), ok, bk, qpos, 0.0, ok, ws, nbytes, T, 0, None)
    assert call(0, ok, None, ok, need - 1) == L.LRKV_ERR_WORKSPACE
    assert call(0, ok, None, None, need) == L.LRKV_ERR_WORKSPACE
    assert call(0, None, None, ok, need) == L.LRKV_ERR_INVALID_ARG       # RoPE needs B^k
    assert call(1, ok, None, ok, need) == L.LRKV_ERR_INVALID_ARG         # absorbed takes no B^k
    assert call(0, ok, None, ok, need, T=0) == L.LRKV_ERR_INVALID_ARG
    assert call(0, ok, None, ok, need, T=5000) == L.LRKV_ERR_INVALID_ARG
    odd = _latent(rank=96)                                                  # not instantiated
    n2 = lib.lrkv_decode_workspace_bytes(0, ctypes.byref(odd), 4096, 0)
    assert call(0, ok, None, ok, n2, desc=odd) == L.LRKV_ERR_UNSUPPORTED
    # workspace grows with the split count and covers every chunk
    assert lib.lrkv_decode_workspace_bytes(0, ctypes.byref(d), 4096, 128) > \
        lib.lrkv_decode_workspace_bytes(0, ctypes.byref(d), 4096, 1)


def test_decode_noalloc_validation(lib):
    """The no-allocation decode rejects, before any device access, a call whose
    workspace would exceed its static scratch, and reports invalid arguments as
    lrkv_decode_attn does."""
    ok = ctypes.c_void_p(FAKE)
    call = lambda mode, desc, T, ns=0, bk=ok, q=ok: lib.lrkv_decode_attn_noalloc(
        mode, ctypes.byref(desc), q, bk, None, 0.0, ok, T, ns, None)
    big = _latent(batch=4, capacity=32768)
    need = lib.lrkv_decode_workspace_bytes(0, ctypes.byref(big), 32768, 1024)
    assert need > L.NOALLOC_SCRATCH_BYTES
    assert call(0, big, 32768, 1024) == L.LRKV_ERR_SCRATCH
    absorbed = _latent(batch=64, capacity=65536)
    assert lib.lrkv_decode_workspace_bytes(1, ctypes.byref(absorbed), 65536, 64) > L.NOALLOC_SCRATCH_BYTES
    assert call(1, absorbed, 65536, 64, bk=None) == L.LRKV_ERR_SCRATCH
    d = _latent()
    assert call(0, d, 0) == L.LRKV_ERR_INVALID_ARG
    assert call(0, d, 4097) == L.LRKV_ERR_INVALID_ARG
    assert call(0, d, 4096, bk=None) == L.LRKV_ERR_INVALID_ARG
    assert call(0, d, 4096, q=None) == L.LRKV_ERR_INVALID_ARG
    assert call(0, _latent(rank=96), 4096) == L.LRKV_ERR_UNSUPPORTED
    assert call(2, _paged(page_size=16), 100, bk=None) == L.LRKV_ERR_UNSUPPORTED
    assert lib.lrkv_decode_attn_noalloc(0, None, ok, ok, None, 0.0, ok, 100, 0, None) == L.LRKV_ERR_INVALID_ARG


def test_paged_validation(lib):
    d = _paged()
    ok = ctypes.c_void_p(FAKE)
    assert lib.lrkv_append_latent(2, ctypes.byref(d), ok, ok, 1, 64 * 32, None) == L.LRKV_ERR_CAPACITY
    assert lib.lrkv_factor_page(ctypes.byref(d), None, 3, None, None, 0, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_factor_page(ctypes.byref(d), ok, -1, None, None, 0, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_factor_page(ctypes.byref(d), ok, 3, ok, None, 64, 0, None) == L.LRKV_ERR_INVALID_ARG
    bad = _paged(page_size=16)
    assert lib.lrkv_factor_page(ctypes.byref(bad), ok, 3, None, None, 0, 0, None) == L.LRKV_ERR_UNSUPPORTED
    # ranks must be multiples of 4 (up to 32), at most 16 query heads per KV head
    for kw in (dict(rank_k=10), dict(rank_v=36), dict(q_per_kv=17), dict(max_pages=65537)):
        bad = _paged(**kw)
        assert lib.lrkv_factor_page(ctypes.byref(bad), ok, 3, None, None, 0, 0, None) == L.LRKV_ERR_UNSUPPORTED, kw
        assert lib.lrkv_decode_workspace_bytes(2, ctypes.byref(bad), 1000, 0) == 0, kw
    assert lib.lrkv_decode_workspace_bytes(2, ctypes.byref(_paged(q_per_kv=16, rank_k=32, rank_v=4)), 1000, 0) > 0
    # int4 factors need their four scale arrays; unknown formats are invalid
    i4 = dict(factor_fmt=1, lk_s=FAKE, rk_s=FAKE, lv_s=FAKE, rv_s=FAKE)
    assert lib.lrkv_decode_workspace_bytes(2, ctypes.byref(_paged(**i4)), 1000, 0) > 0
    assert lib.lrkv_decode_workspace_bytes(2, ctypes.byref(_paged(**dict(i4, rv_s=None))), 1000, 0) == 0
    assert lib.lrkv_decode_workspace_bytes(2, ctypes.byref(_paged(factor_fmt=2)), 1000, 0) == 0
    bad = _paged(**dict(i4, lk_s=None))
    assert lib.lrkv_factor_page(ctypes.byref(bad), ok, 3, None, None, 0, 0, None) == L.LRKV_ERR_INVALID_ARG
    need = lib.lrkv_decode_workspace_bytes(2, ctypes.byref(d), 1000, 0)
    assert need > 0
    assert lib.lrkv_decode_attn(2, ctypes.byref(d), ok, ok, None, 0.0, ok, ok, need, 1000, 0, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_decode_attn(2, ctypes.byref(d), ok, None, None, 0.0, ok, ok, need - 4, 1000, 0, None) == L.LRKV_ERR_WORKSPACE


def _plan(lib, d, lens, n_new):
    lens = np.asarray(lens, np.int32)
    n = lib.lrkv_paged_plan(ctypes.byref(d), lens.ctypes.data, n_new, None, 0)
    out = np.zeros((max(n, 1), 3), np.int32)
    got = lib.lrkv_paged_plan(ctypes.byref(d), lens.ctypes.data, n_new, out.ctypes.data, n)
    assert got == n
    return out[:n]


def test_paged_plan_matches_oracle_page_states(lib):
    """The pages the planner schedules are exactly those the oracle's closed form
    turns factored between length len and len + n_new."""
    d = _paged(batch=3, kv_heads=2, max_pages=80)
    rng = np.random.default_rng(0)
    for _ in range(60):
        lens = rng.integers(0, 60 * 32, 3)
        n_new = int(rng.choice([1, 1, 1, 32, 33, 500]))
        plan = _plan(lib, d, lens, n_new)
        expect = []
        for b in range(3):
            before = opaged.page_table(lens[b], 32, 1, 4) if lens[b] else np.zeros(0, np.int32)
            after = opaged.page_table(lens[b] + n_new, 32, 1, 4)
            newly = [p for p in range(len(after)) if after[p] >= 0 and (p >= len(before) or before[p] < 0)]
            for h in range(2):
                expect += [(b, h, p) for p in newly]
        assert [tuple(r) for r in plan] == expect
    # prefill of the hybrid workload: 1019 pages per (b, h)
    d5 = _paged(batch=8, kv_heads=8, max_pages=1024)
    assert lib.lrkv_paged_plan(ctypes.byref(d5), np.zeros(8, np.int32).ctypes.data, 32768, None, 0) == 8 * 8 * 1019
    assert lib.lrkv_paged_plan(ctypes.byref(d5), np.zeros(8, np.int32).ctypes.data, 32769 + 1024 * 32, None, 0) < 0


def test_workspace_monotone_in_length(lib):
    """A workspace sized for a length serves every shorter length (any split count)."""
    for mode in (0, 1):
        d = _latent(capacity=70000 // 32 * 32)
        prev = 0
        for T in list(range(1, 3000, 37)) + list(range(65000, 69000, 33)):
            for ns in (0, 1, 7, 64):
                n = lib.lrkv_decode_workspace_bytes(mode, ctypes.byref(d), T, ns)
                assert n > 0
            n = lib.lrkv_decode_workspace_bytes(mode, ctypes.byref(d), T, 0)
            assert n >= prev
            prev = n
    d = _paged(max_pages=2000)
    prev = 0
    for T in range(1, 64000, 311):
        n = lib.lrkv_decode_workspace_bytes(2, ctypes.byref(d), T, 0)
        assert n >= prev
        prev = n


def test_probe_stream_read_validation(lib):
    ok = ctypes.c_void_p(FAKE)
    bad = ctypes.c_void_p(FAKE + 8)
    assert lib.lrkv_probe_stream_read(None, 1024, ok, 4, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_probe_stream_read(ok, 1000, ok, 4, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_probe_stream_read(bad, 1024, ok, 4, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_probe_stream_read(ok, 1024, None, 4, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_probe_stream_read(ok, 1024, ok, 0, None) == L.LRKV_ERR_INVALID_ARG


def test_projection_validation(lib):
    ok = ctypes.c_void_p(FAKE)
    need = lib.lrkv_project_workspace_bytes(4, 4096, 8192)
    assert need >= 4 * 4096 * 4
    assert lib.lrkv_project_workspace_bytes(4, 4096, 8190) == 0       # K not a multiple of 32
    assert lib.lrkv_project_workspace_bytes(4, 4100, 8192) == 0       # N not a multiple of 16
    assert lib.lrkv_project_workspace_bytes(0, 4096, 8192) == 0
    # latent projection: x [n][d], a_t [U r][d], h [n][U][r]
    assert lib.lrkv_latent_project(None, 4, 4096, ok, 8, 256, ok, ok, 1 << 30, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_latent_project(ok, 4, 4096, ok, 1, 250, ok, ok, 1 << 30, None) == L.LRKV_ERR_UNSUPPORTED
    assert lib.lrkv_latent_project(ok, 4, 4001, ok, 8, 256, ok, ok, 1 << 30, None) == L.LRKV_ERR_UNSUPPORTED
    ws = lib.lrkv_project_workspace_bytes(4, 8 * 256, 4096)
    assert lib.lrkv_latent_project(ok, 4, 4096, ok, 8, 256, ok, ok, ws - 4, None) == L.LRKV_ERR_WORKSPACE
    assert lib.lrkv_latent_project(ok, 4, 4096, ok, 8, 256, ok, None, ws, None) == L.LRKV_ERR_WORKSPACE
    # output projection: o [B][Hq][r], w_t [d][Hq r], y [B][d]
    assert lib.lrkv_output_project(ok, 0, 32, 256, ok, 4096, ok, ok, need, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_output_project(ok, 4, 32, 256, None, 4096, ok, ok, need, None) == L.LRKV_ERR_INVALID_ARG
    assert lib.lrkv_output_project(ok, 4, 32, 256, ok, 4095, ok, ok, need, None) == L.LRKV_ERR_UNSUPPORTED
    assert lib.lrkv_output_project(ok, 4, 32, 256, ok, 4096, ok, ok, need - 4, None) == L.LRKV_ERR_WORKSPACE


def test_prefill_validation(lib):
    d = _latent()
    ok = ctypes.c_void_p(FAKE)
    need = lib.lrkv_prefill_workspace_bytes(ctypes.byref(d), 512, 4096)
    assert need >= 512 * 32 * 128 * 4
    assert lib.lrkv_prefill_workspace_bytes(ctypes.byref(d), 0, 4096) == 0
    assert lib.lrkv_prefill_workspace_bytes(ctypes.byref(d), 512, 4097) == 0        # beyond capacity
    i4 = _latent(fmt=1, sk=FAKE, sv=FAKE)
    assert lib.lrkv_prefill_workspace_bytes(ctypes.byref(i4), 512, 4096) == 0       # int4 latents
    call = lambda desc, q=ok, m=512, hml=4096, ws=need, out=ok: lib.lrkv_prefill_attn(
        ctypes.byref(desc), q, ok, ok, m, hml, 0.0, out, ok, ws, None)
    assert call(d, q=None) == L.LRKV_ERR_INVALID_ARG
    assert call(d, out=ctypes.c_void_p(FAKE + 4)) == L.LRKV_ERR_INVALID_ARG
    assert call(d, m=0) == L.LRKV_ERR_INVALID_ARG
    assert call(d, hml=4097) == L.LRKV_ERR_INVALID_ARG
    assert call(d, ws=need - 1) == L.LRKV_ERR_WORKSPACE
    assert call(i4) == L.LRKV_ERR_UNSUPPORTED
    assert call(_latent(rank=128)) == L.LRKV_ERR_UNSUPPORTED
    assert call(_latent(head_dim=64)) == L.LRKV_ERR_UNSUPPORTED


def test_decode_step_validation(lib):
    """lrkv_decode_step rejects before enqueueing: the append's checks (capacity,
    pointers, alignment), then the decode's (queries, workspace for the length after
    the append)."""
    d = _latent(batch=1, units=8, kv_per_unit=4, rank=256, capacity=4096)
    ok = ctypes.c_void_p(FAKE)
    need = lib.lrkv_decode_workspace_bytes(0, ctypes.byref(d), 4001, 0)
    assert need > 0
    args = lambda **kw: dict(dict(mode=0, nk=ok, nv=ok, n=1, q=ok, bk=ok, out=ok, ws=ok, wsb=need, hml=4000), **kw)
    def call(**kw):
        a = args(**kw)
        return lib.lrkv_decode_step(a["mode"], ctypes.byref(d), a["nk"], a["nv"], a["n"], a["q"], a["bk"], None,
                                    0.0, a["out"], a["ws"], a["wsb"], a["hml"], 0, None)
    assert call(hml=4096) == L.LRKV_ERR_CAPACITY
    assert call(hml=4095, n=2) == L.LRKV_ERR_CAPACITY
    assert call(n=0) == L.LRKV_ERR_INVALID_ARG
    assert call(nk=None) == L.LRKV_ERR_INVALID_ARG
    assert call(nk=ctypes.c_void_p(FAKE + 4)) == L.LRKV_ERR_INVALID_ARG
    assert call(q=None) == L.LRKV_ERR_INVALID_ARG
    assert call(bk=None) == L.LRKV_ERR_INVALID_ARG
    assert call(out=None) == L.LRKV_ERR_INVALID_ARG
    assert call(mode=7) == L.LRKV_ERR_INVALID_ARG
    assert call(ws=None) == L.LRKV_ERR_WORKSPACE
    assert call(wsb=need - 1) == L.LRKV_ERR_WORKSPACE
    # absorbed mode takes no B^k
    assert call(mode=1) == L.LRKV_ERR_INVALID_ARG
