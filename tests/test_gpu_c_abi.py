"""The routing path driven from a C program through the C ABI alone
(tests/helpers/abi_pipeline, built by build(): HIP runtime calls for memory,
copies and one stream; tk_route -> tk_map -> tk_expand_quant (1x128 FP8) ->
tk_reduce or tk_reduce_dense on the device; no Python, no torch).  The test
writes seeded inputs as raw files, runs the program and compares every
output with the oracle's chain on the same inputs: indices, counts, offsets,
positions, row sources, codes and scales bit for bit, weights within the
weight tolerance, the combine within the combine tolerance.

Cases: the DeepSeek-V3 gating (sigmoid + bias, 8 groups, top-4 groups,
x2.5) at T=1000, H=1024 with tk_reduce and at T=4500, H=2048 with
tk_reduce_dense (its staged form: two rounds of 9-token workgroups); a masked
share (softmax, experts [16, 40) of 64 local, k=6) at T=777; and the tiny
softmax top-2 configuration.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle
from moe_routing_amd import synth
from tk_testutil import W_ATOL, W_RTOL, combine_report

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "helpers", "abi_pipeline")

SOFTMAX, SIGMOID = 0, 1

CASES = {
    "v3_T1000": dict(T=1000, E=256, k=8, H=1024, route=synth.ROUTE_V3, bias=True, local=None,
                     dense=0),
    "v3_T4500_dense": dict(T=4500, E=256, k=8, H=2048, route=synth.ROUTE_V3, bias=True,
                           local=None, dense=1),
    "masked_softmax": dict(T=777, E=64, k=6, H=512, local=(16, 40), bias=False, dense=0,
                           route=dict(score=SOFTMAX, n_groups=1, topk_groups=1, group_topn=0,
                                      renormalize=1, route_scale=1.0)),
    "tiny": dict(T=64, E=16, k=2, H=256, route=synth.ROUTE_TINY, bias=False, local=None,
                 dense=0),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_c_program_runs_the_path(name, tmp_path):
    assert os.path.exists(EXE), "tests/helpers/abi_pipeline is missing: run build() first"
    c = CASES[name]
    T, E, k, H = c["T"], c["E"], c["k"], c["H"]
    lo, hi = c["local"] or (0, E)
    r = c["route"]
    rng = np.random.default_rng(sum(map(ord, name)))
    logits = synth.normal_f32(rng, (T, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32) if c["bias"] else None
    x = synth.normal_bf16(rng, (T, H))
    y = synth.normal_bf16(rng, (T * k, H))
    logits.tofile(tmp_path / "logits")
    x.tofile(tmp_path / "x")
    y.tofile(tmp_path / "y")
    if bias is not None:
        bias.tofile(tmp_path / "bias")
    args = [EXE, str(tmp_path), T, E, k, H, r["score"], r["n_groups"], r["topk_groups"],
            r["group_topn"], repr(float(r["route_scale"])), lo, hi, int(bias is not None),
            c["dense"]]
    print(f"abi_pipeline {name}: {' '.join(map(str, args[2:]))}", flush=True)
    run = subprocess.run([str(a) for a in args], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0, run.stderr

    def got(fname, dtype, shape):
        return np.fromfile(tmp_path / fname, dtype=dtype).reshape(shape)

    cap, nl = T * k, hi - lo
    o_idx, o_w = oracle.route(logits, bias, k, **r)
    assert np.array_equal(got("idx", np.int32, (T, k)), o_idx)
    assert np.allclose(got("w", np.float32, (T, k)), o_w, rtol=W_RTOL, atol=W_ATOL)
    oc, oo, op, ors = oracle.map_routes(o_idx, E, lo, hi)
    R = int(oo[-1])
    assert np.array_equal(got("counts", np.int32, (nl,)), oc)
    assert np.array_equal(got("offsets", np.int32, (nl + 1,)), oo)
    assert np.array_equal(got("pos", np.int32, (T, k)), op)
    assert np.array_equal(got("row_src", np.int32, (cap,))[:R], ors)
    o_xq, o_sc = oracle.expand(x, op, 1, cap)
    assert np.array_equal(got("xq", np.uint8, (cap, H))[:R], o_xq[:R])
    assert np.array_equal(got("scales", np.float32, (cap, H // 128))[:R], o_sc[:R])
    rep = combine_report(got("out", np.uint16, (T, H)),
                         oracle.reduce(y, op, o_w.astype(np.float32)))
    print(f"abi_pipeline {name}: combine {rep}")
    assert rep["ok"], rep
    if c["local"] is not None:
        assert R < cap and (op < 0).all(1).any(), "the mask should leave tokens without rows"
