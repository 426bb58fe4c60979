"""The C ABI's host-side validation under AddressSanitizer (CPU only).

The library is built a second time with its host code instrumented
(`python -m rank_sgmv_bgmv_amd.build --asan`), and tests/test_abi.py -- every
declared symbol, every documented status for bad arguments, workspace sizing
-- runs against it in a child process started with the sanitizer runtime
preloaded.  Any heap or stack overflow, use after free or bad free in the
argument checks, the workspace layout or the launch configuration fails the
child.  No call here reaches a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)

CHILD = """
import sys
sys.path.insert(0, {root!r}); sys.path.insert(0, {tests!r})
import pytest
import rank_sgmv_bgmv_amd as L
L.LIB_PATH = {lib!r}
sys.exit(pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}]))
"""


@pytest.mark.timeout(600)
def test_abi_checks_under_address_sanitizer():
    if not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    from rank_sgmv_bgmv_amd import build
    lib = build.build(asan=True)
    runtime = build.asan_runtime()
    if not os.path.exists(runtime):
        pytest.skip(f"AddressSanitizer runtime not found at {runtime}")
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    code = CHILD.format(root=ROOT, tests=HERE, lib=lib, abi=os.path.join(HERE, "test_abi.py"))
    p = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=540)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out, out[-4000:]
    assert " passed" in p.stdout
