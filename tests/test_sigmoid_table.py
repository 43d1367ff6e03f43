"""The bf16 sigmoid table that the build writes (it is compiled into the
SwiGLU kernels) against the oracle's pinned sigmoid, on every bf16 value.

The table holds, interleaved by sign, the sigmoid of each bf16 magnitude in a
band, plus one entry below the band (every smaller magnitude: 1/2) and one
above it (every larger magnitude, infinities and NaNs included: 1 for
positive, 0 for negative arguments).  The lookup rule is restated here from
that description: i = clamp(m, lo - 1, hi) - (lo - 1), entry 2 i + sign.
"""
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INC = os.path.join(ROOT, "_build", "sigmoid_table.inc")
HDR = os.path.join(ROOT, "moe_routing_amd", "csrc", "sigmoid_table.h")


def _band():
    txt = open(HDR).read()
    get = lambda name: int(txt.split(f"{name} = ")[1].split("u;")[0], 16)
    return get("kSigLo"), get("kSigHi")


def _table():
    if not os.path.exists(INC):
        pytest.skip("library not built (the build writes the table)")
    body = open(INC).read().split("\n", 1)[1]
    return np.array([float.fromhex(t.strip()[:-1]) for t in body.replace("\n", " ").split(",")
                     if t.strip()], np.float32)


def test_table_is_the_pinned_sigmoid_on_every_bf16_value():
    lo, hi = _band()
    tab = _table()
    assert tab.size == 2 * (hi - lo + 2)
    bits = np.arange(0x10000, dtype=np.uint32)
    g = (bits << 16).view(np.float32)
    m, sgn = bits & 0x7FFF, bits >> 15
    i = np.clip(m, lo - 1, hi) - (lo - 1)
    lut = tab[2 * i + sgn]
    ref = oracle.sigmoid_f32(g)
    ok = ~np.isnan(g)
    assert np.array_equal(lut[ok].view(np.uint32), ref[ok].view(np.uint32))
    # the constant entries: 1/2 below the band, 1 / 0 above it
    assert tab[0] == 0.5 and tab[1] == 0.5
    assert tab[-2] == 1.0 and tab[-1] == 0.0
