"""Host proof of the FP4 kernel's E2M1 encoder.

The kernel rounds |v| (clamped to 6, the range below 1 shifted by +1.0) to one
mantissa bit with integer arithmetic on the fp32 bits.  The helper enumerates
every value the kernel encodes -- each finite bf16 input times each power of
two a block scale can take -- and requires the result to equal the nearest
E2M1 value with ties to the even code, found by plain search.  This checks the
kernel's arithmetic, not the oracle.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_e2m1_encoder_equals_nearest_even_on_domain():
    src = os.path.join(HERE, "helpers", "e2m1_domain.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "e2m1")
        subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", src, "-o", exe, "-lm"],
                       check=True, capture_output=True)
        r = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=300)
    n, bad = map(int, r.stdout.strip().splitlines()[-1].split())
    assert n > 5_000_000, r.stdout
    assert bad == 0, r.stdout
