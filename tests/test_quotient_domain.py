"""Host proof of the FP8 expand kernel's division shortcut.

The kernel replaces x/scale by Markstein's correction of x*RN(1/scale),
with the residual formed negated so that x = -0 keeps its sign.  The
helper enumerates every (x, scale) pair the kernel can see -- scale from every
bf16 block maximum >= 1e-4 (and the 1e-4 clamp), x every bf16 value up to
that maximum -- and requires the shortcut to equal the IEEE quotient bit for
bit except where both lie below 2^-10 (they then encode to the same E4M3
signed zero; such pairs only occur near the bottom of the fp32 range).  This checks the
kernel's arithmetic, not the oracle.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_markstein_quotient_equals_ieee_division_on_domain():
    src = os.path.join(HERE, "helpers", "quotient_domain.c")
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "qd")
        base = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-mfma", src, "-o", exe, "-lm"]
        try:
            subprocess.run(base[:1] + ["-fopenmp"] + base[1:], check=True, capture_output=True)
        except subprocess.CalledProcessError:
            subprocess.run(base, check=True, capture_output=True)
        env = dict(os.environ, OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS", "8"))
        r = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=600, env=env)
    pairs, bad, tiny = map(int, r.stdout.strip().splitlines()[-1].split())
    assert pairs > 400_000_000, r.stdout
    assert bad == 0, r.stdout             # equal wherever the FP8 code depends on it
    assert tiny < pairs // 1000, r.stdout   # both below 2^-10: both encode to zero
