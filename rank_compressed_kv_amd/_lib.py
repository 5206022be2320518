"""ctypes view of liblrkv.so (include/lrkv.h). Loading fails loudly when the
library has not been built: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# LRKV_LIBRARY selects another build of the same library (e.g. the host-checked
# one); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("LRKV_LIBRARY") or os.path.join(_HERE, "liblrkv.so")

LRKV_OK = 0
LRKV_ERR_INVALID_ARG = -1
LRKV_ERR_UNSUPPORTED = -2
LRKV_ERR_CAPACITY = -3
LRKV_ERR_WORKSPACE = -4
LRKV_ERR_HIP = -5
LRKV_ERR_SCRATCH = -6

NOALLOC_SCRATCH_BYTES = 16 << 20      # LRKV_NOALLOC_SCRATCH_BYTES

FMT_FP16 = 0
FMT_INT4_G32 = 1

MODE_ROPE_RECON = 0
MODE_ABSORBED = 1
MODE_HYBRID_PAGED = 2

PAGE_EMPTY = -(2 ** 31)
BLOCK = 32

EXPORTS = (
    "lrkv_status_string", "lrkv_version", "lrkv_decode_workspace_bytes", "lrkv_append_latent",
    "lrkv_decode_attn", "lrkv_decode_prepare", "lrkv_decode_partials", "lrkv_merge_partials",
    "lrkv_factor_page", "lrkv_paged_plan", "lrkv_project_workspace_bytes", "lrkv_latent_project",
    "lrkv_output_project", "lrkv_probe_stream_read", "lrkv_prefill_workspace_bytes", "lrkv_prefill_attn",
    "lrkv_decode_attn_noalloc", "lrkv_decode_step",
)

c_i32 = ctypes.c_int32
c_vp = ctypes.c_void_p


class LatentCacheDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("units", c_i32), ("kv_per_unit", c_i32), ("q_per_kv", c_i32),
        ("head_dim", c_i32), ("rank", c_i32), ("capacity", c_i32), ("fmt", c_i32),
        ("rope_theta", ctypes.c_float),
        ("hk", c_vp), ("hv", c_vp), ("sk", c_vp), ("sv", c_vp), ("lens", c_vp),
    ]


class PagedCacheDesc(ctypes.Structure):
    _fields_ = [
        ("batch", c_i32), ("kv_heads", c_i32), ("q_per_kv", c_i32), ("head_dim", c_i32),
        ("page_size", c_i32), ("sink_pages", c_i32), ("window_pages", c_i32),
        ("rank_k", c_i32), ("rank_v", c_i32), ("max_pages", c_i32),
        ("dense_k", c_vp), ("dense_v", c_vp), ("lk", c_vp), ("rk", c_vp), ("lv", c_vp), ("rv", c_vp),
        ("page_table", c_vp), ("lens", c_vp),
        ("factor_fmt", c_i32), ("lk_s", c_vp), ("rk_s", c_vp), ("lv_s", c_vp), ("rv_s", c_vp),
    ]


class LrkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m rank_compressed_kv_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        L.lrkv_status_string.argtypes = [c_i32]
        L.lrkv_status_string.restype = ctypes.c_char_p
        L.lrkv_version.argtypes = []
        L.lrkv_version.restype = c_i32
        L.lrkv_decode_workspace_bytes.argtypes = [c_i32, c_vp, c_i32, c_i32]
        L.lrkv_decode_workspace_bytes.restype = ctypes.c_size_t
        L.lrkv_append_latent.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_vp]
        L.lrkv_append_latent.restype = c_i32
        L.lrkv_decode_attn.argtypes = [c_i32, c_vp, c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_vp,
                                       ctypes.c_size_t, c_i32, c_i32, c_vp]
        L.lrkv_decode_attn.restype = c_i32
        L.lrkv_decode_step.argtypes = [c_i32, c_vp, c_vp, c_vp, c_i32, c_vp, c_vp, c_vp, ctypes.c_float, c_vp,
                                       c_vp, ctypes.c_size_t, c_i32, c_i32, c_vp]
        L.lrkv_decode_step.restype = c_i32
        L.lrkv_decode_attn_noalloc.argtypes = [c_i32, c_vp, c_vp, c_vp, c_vp, ctypes.c_float, c_vp, c_i32, c_i32,
                                               c_vp]
        L.lrkv_decode_attn_noalloc.restype = c_i32
        L.lrkv_decode_prepare.argtypes = [c_i32, c_vp, c_vp, c_vp, c_vp, ctypes.c_float, c_vp,
                                          ctypes.c_size_t, c_i32, c_i32, c_vp]
        L.lrkv_decode_prepare.restype = c_i32
        L.lrkv_decode_partials.argtypes = [c_i32, c_vp, c_vp, ctypes.c_float, c_vp, ctypes.c_size_t,
                                           c_i32, c_i32, c_vp]
        L.lrkv_decode_partials.restype = c_i32
        L.lrkv_merge_partials.argtypes = [c_i32, c_vp, c_vp, c_vp, ctypes.c_size_t, c_i32, c_i32, c_vp]
        L.lrkv_merge_partials.restype = c_i32
        L.lrkv_factor_page.argtypes = [ctypes.POINTER(PagedCacheDesc), c_vp, c_i32, c_vp, c_vp,
                                       c_i32, c_i32, c_vp]
        L.lrkv_factor_page.restype = c_i32
        L.lrkv_paged_plan.argtypes = [ctypes.POINTER(PagedCacheDesc), c_vp, c_i32, c_vp, c_i32]
        L.lrkv_paged_plan.restype = c_i32
        L.lrkv_project_workspace_bytes.argtypes = [c_i32, c_i32, c_i32]
        L.lrkv_project_workspace_bytes.restype = ctypes.c_size_t
        L.lrkv_latent_project.argtypes = [c_vp, c_i32, c_i32, c_vp, c_i32, c_i32, c_vp, c_vp, ctypes.c_size_t, c_vp]
        L.lrkv_latent_project.restype = c_i32
        L.lrkv_output_project.argtypes = [c_vp, c_i32, c_i32, c_i32, c_vp, c_i32, c_vp, c_vp, ctypes.c_size_t, c_vp]
        L.lrkv_output_project.restype = c_i32
        L.lrkv_probe_stream_read.argtypes = [c_vp, ctypes.c_size_t, c_vp, c_i32, c_vp]
        L.lrkv_probe_stream_read.restype = c_i32
        L.lrkv_prefill_workspace_bytes.argtypes = [ctypes.POINTER(LatentCacheDesc), c_i32, c_i32]
        L.lrkv_prefill_workspace_bytes.restype = ctypes.c_size_t
        L.lrkv_prefill_attn.argtypes = [ctypes.POINTER(LatentCacheDesc), c_vp, c_vp, c_vp, c_i32, c_i32,
                                        ctypes.c_float, c_vp, c_vp, ctypes.c_size_t, c_vp]
        L.lrkv_prefill_attn.restype = c_i32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().lrkv_status_string(status).decode()


def check(status: int, where: str) -> int:
    if status < 0:
        raise LrkvError(status, where)
    return status
