"""Host proof of the FP4 kernel's E2M1 encoding.

The kernel reads each code from a compile-time table indexed by the
quotient's clamped bf16 magnitude (moe_routing_amd/csrc/e2m1_table.h).  The
helper includes that header and enumerates every value the kernel encodes --
each finite bf16 input times each power of two a block scale can take -- and
requires the lookup to equal the nearest E2M1 value with ties to the even
code, found by plain search.  This checks the kernel's table and lookup, not
the oracle.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


CSRC = os.path.join(os.path.dirname(HERE), "moe_routing_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_e2m1_encoder_equals_nearest_even_on_domain():
    src = os.path.join(HERE, "helpers", "e2m1_domain.cpp")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "e2m1")
        subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-I", CSRC, src, "-o", exe],
                       check=True, capture_output=True)
        r = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=300)
    n, bad = map(int, r.stdout.strip().splitlines()[-1].split())
    assert n > 5_000_000, r.stdout
    assert bad == 0, r.stdout
