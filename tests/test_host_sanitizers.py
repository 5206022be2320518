"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

A copy of liblrkv.so is built with both sanitizers on its host code
and the C-ABI tests (argument validation, status strings, the paged planner,
the workspace sizing) run against it in a child interpreter with the ASan
runtime preloaded. Any sanitizer report ends the child with a non-zero status
and fails this test. No GPU is needed or touched: no call there reaches a
kernel launch."""
import os
import subprocess
import sys

import pytest

from rank_compressed_kv_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def checked_lib(tmp_path_factory):
    try:
        B.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    out = tmp_path_factory.mktemp("host_checked")
    return B.build_host_checked(str(out), verbose=False)


def test_abi_suite_under_host_sanitizers(checked_lib):
    env = B.host_checked_env(checked_lib)
    env["PYTHONPATH"] = ROOT + (os.pathsep + env["PYTHONPATH"] if env.get("PYTHONPATH") else "")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
           os.path.join(ROOT, "tests", "test_abi.py")]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    report = res.stdout[-4000:] + res.stderr[-4000:]
    assert res.returncode == 0, report
    assert "passed" in res.stdout and "AddressSanitizer" not in report and "runtime error" not in report, report


def test_host_checked_library_is_the_one_loaded(checked_lib):
    """The build is instrumented, and the child really loads it (not the in-tree one)."""
    syms = subprocess.run(["nm", "-D", "--undefined-only", checked_lib], capture_output=True, text=True)
    if syms.returncode == 0:
        assert "__asan_report" in syms.stdout and "__ubsan_handle" in syms.stdout
    env = B.host_checked_env(checked_lib)
    env["PYTHONPATH"] = ROOT
    code = ("from rank_compressed_kv_amd import _lib as L; import sys; L.lib(); "
            "maps = open('/proc/self/maps').read(); "
            "sys.exit(0 if L.LIB_PATH in maps and 'asan' in maps else 3)")
    res = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=300)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-2000:]
