"""The boundary checks under AddressSanitizer (CPU only).

tests/test_boundary.py is run in a child process against libtk built with
AddressSanitizer on its host code (argument checks, the error state behind
tk_last_error, launch wrappers; device code built as usual), with the
compiler's ASan runtime preloaded.  Every call there returns before any
device work, so this runs without a GPU.  The child must pass and ASan must
report nothing.
"""
import os
import subprocess
import sys

import pytest

from moe_routing_amd import _build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_boundary_checks_are_clean_under_asan():
    if not os.path.exists(_build.ASAN_LIB):
        _build.build_asan()
    rt = _build.asan_runtime()
    if rt is None:
        pytest.skip("the compiler's ASan runtime is not installed")
    env = dict(os.environ)
    # the ASan runtime must come first among the preloaded libraries; any that
    # are already listed stay
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:exitcode=86"
    env["TK_BOUNDARY_LIB"] = _build.ASAN_LIB
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_boundary.py"), "-k",
                        "not calibration and not bench_refuses and not product_path"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
