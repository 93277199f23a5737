"""The library's host code under AddressSanitizer: the C ABI checks of
test_abi.py (shape validation, workspace planning and regions, argument checks,
the error paths of every entry point) rerun in a child process against the
build with the sanitizer on its host pass (GPU code cannot be built with it
here: device-side AddressSanitizer needs XNACK).  Nothing here uses a GPU."""
import os
import subprocess
import sys

import pytest

pytest.importorskip("torch")


def test_abi_checks_pass_under_host_address_sanitizer():
    from kv_reuse_amd import build
    lib = build.build_asan_host()
    rt = build.asan_runtime()
    here = os.path.dirname(os.path.abspath(__file__))
    # the sanitizer's runtime must come first among the preloaded libraries
    pre = os.environ.get("LD_PRELOAD", "")
    env = dict(os.environ, HS2_LIBRARY=lib, LD_PRELOAD=rt + (":" + pre if pre else ""),
               ASAN_OPTIONS="detect_leaks=0")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(here, "test_abi.py"), "-q",
                        "-p", "no:cacheprovider", "-m", "not gpu"],
                       env=env, capture_output=True, text=True, timeout=900,
                       cwd=os.path.dirname(here))
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in p.stdout
