"""Build liblrkv.so (HIP, gfx950) in-tree: rank_compressed_kv_amd/liblrkv.so.

Every .hip source under csrc/ is compiled by hipcc for gfx950 only, with packed
fp32 arithmetic disabled, and linked into one shared library with a plain C ABI
(include/lrkv.h). Run ``python -m rank_compressed_kv_amd.build``.

``python -m rank_compressed_kv_amd.build --host-checked DIR`` builds a second
copy of the library (device code at -O1) whose host code carries
AddressSanitizer and UndefinedBehaviorSanitizer, for checking the C ABI's
argument validation and planning on a machine without a GPU. Load it with LRKV_LIBRARY=DIR/liblrkv.so
and the clang ASan runtime preloaded (host_checked_env gives the environment).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
INC = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "liblrkv.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INC, "-I" + SRC,
]
# Per-source extras: MFMA accumulators in the arithmetic registers, so that
# operands resident for a whole loop (Q' of the head-wave kernel; B^k fragments
# and queries of the prefill kernel), pinned to the AGPRs, are read by the MFMAs
# in place, and the vector work on the accumulators needs no copies.
FILE_FLAGS = {
    "rope_decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stderr}")
    noise = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if noise.strip():
        sys.stderr.write(noise + "\n")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(_compile, sources))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    shutil.move(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# Host sanitizers: every -fsanitize option applies to the host pass only.
HOST_CHECK = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
              "-Xarch_host", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
CLANGXX = os.environ.get("CLANGXX", "/opt/rocm/llvm/bin/clang++")
ASAN_RT = "/opt/rocm/llvm/lib/clang/{v}/lib/linux/libclang_rt.asan-x86_64.so"


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that the host-checked build needs."""
    found = sorted(glob.glob(ASAN_RT.format(v="*")))
    if not found:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    return found[-1]


def build_host_checked(out_dir: str, verbose: bool = True) -> str:
    """Sanitizer-instrumented (host code) liblrkv.so in out_dir (see the module docstring)."""
    os.makedirs(out_dir, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(SRC, "*.hip")))

    def one(src: str) -> str:
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++17",
               "-I" + INC, "-I" + SRC, *HOST_CHECK, "-c", src, "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc (host-checked) failed for {src}:\n{res.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(sources))) as ex:
        objs = list(ex.map(one, sources))
    out = os.path.join(out_dir, "liblrkv.so")
    # Host objects only: the link is a plain clang++ link against the HIP runtime.
    cmd = [CLANGXX, "-shared", "-fsanitize=address,undefined", "-shared-libsan", *objs,
           "-L/opt/rocm/lib", "-lamdhip64", "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"host-checked link failed:\n{res.stderr}")
    if verbose:
        print(f"built {out}")
    return out


def host_checked_env(lib_path: str, base: dict | None = None) -> dict:
    """Environment that loads the host-checked library: ASan runtime preloaded
    ahead of anything already preloaded, leak checking off (the interpreter and
    the HIP runtime keep allocations until exit), first error fatal."""
    env = dict(os.environ if base is None else base)
    pre = env.get("LD_PRELOAD", "")
    env["LD_PRELOAD"] = asan_runtime() + (":" + pre if pre else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    env["LRKV_LIBRARY"] = lib_path
    return env


if __name__ == "__main__":
    if len(sys.argv) == 3 and sys.argv[1] == "--host-checked":
        build_host_checked(sys.argv[2])
    else:
        build()
