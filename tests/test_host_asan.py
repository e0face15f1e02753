"""Host AddressSanitizer run of the C ABI's validation layer.

The host code of libppattn (argument checks, overlap and alignment checks,
workspace sizing, error strings, plan and launch set-up) is built with ASan
(shared_prefix_stream_amd.build.build_host_asan), and the ABI tests of
test_abi_cpu.py run against that build in a child process that loads the
ASan runtime first.  No GPU is used: every call those tests make is rejected
on the host or only sizes a workspace."""
import os
import subprocess
import sys

import pytest

from shared_prefix_stream_amd import build as ppbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_validation_under_host_asan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("a library is already preloaded in this environment; the ASan runtime must come first")
    try:
        ppbuild._hipcc()
        runtime = ppbuild.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = ppbuild.build_host_asan(str(tmp_path / "libppattn_asan.so"), str(tmp_path / "obj"))
    env = dict(os.environ, PP_ATTN_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:verify_asan_link_order=0")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    report = r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stdout + r.stderr, report
    assert r.returncode == 0, report
    assert " passed" in r.stdout, report
