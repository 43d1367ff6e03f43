"""End-to-end GPU pipelines against the CPU oracle: each step's GPU output
feeds the next GPU step, and every stage is compared with the oracle run on
the same inputs.

tiny      T=64, E=16, k=2, H=256: softmax top-2, bf16 expand, reduce.
ep_share  T=32768, H=7168, E=256, k=8, one expert-parallel rank's share
          (experts 32..63 local), v3 gating with a log-Zipf popularity offset:
          route, map with the local mask, FP8 expand, stand-in expert
          (dequantise * 0.5), reduce -- all full size on the GPU, every
          output compared in full with the oracle's chain on the same inputs.
v3        the benchmarked step at T=8192, H=7168, E=256 (8 groups of 32),
          k=8: sigmoid + bias gating, map, FP8 expand of hidden states with
          outlier rows, tk_reduce_dense of (65536, 7168) expert outputs -- in
          full against the oracle's chain.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import W_ATOL, W_RTOL, combine_report, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def test_pipeline_tiny():
    cfg = synth.tiny(0)
    T, E, k, H = cfg["T"], cfg["E"], cfg["k"], cfg["H"]
    r = cfg["route"]
    idx, w = tk.tk_route(to_dev(cfg["logits"]), None, k, tk.RouteOpts(**r))
    counts, offsets, pos, row_src = tk.tk_map(idx, E)
    xe, _ = tk.tk_expand_quant(to_dev(cfg["x"], bf16=True), pos, tk.TK_EXPAND_BF16, T * k)
    out = tk.tk_reduce(to_dev(cfg["y"], bf16=True), pos, w)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route(cfg["logits"], None, k, **r)
    oc, oo, op, ors = oracle.map_routes(o_idx, E)
    assert np.array_equal(to_host(idx), o_idx)
    assert np.allclose(to_host(w), o_w, rtol=W_RTOL, atol=W_ATOL)
    assert np.array_equal(to_host(pos), op) and np.array_equal(to_host(row_src), ors)
    assert np.array_equal(to_host(xe), oracle.expand(cfg["x"], op, 0, T * k)[0])
    rep = combine_report(to_host(out), oracle.reduce(cfg["y"], op, o_w.astype(np.float32)))
    assert rep["ok"], rep


@pytest.mark.slow
def test_pipeline_ep_share():
    cfg = synth.ep_share(0)
    T, E, k, H = cfg["T"], cfg["E"], cfg["k"], cfg["H"]
    lo, hi = cfg["local"]
    r = cfg["route"]
    x_d = to_dev(cfg["x"], bf16=True)
    idx, w = tk.tk_route(to_dev(cfg["logits"]), None, k, tk.RouteOpts(**r))
    counts, offsets, pos, row_src = tk.tk_map(idx, E, lo, hi)
    cap = T * k
    xq, sc = tk.tk_expand_quant(x_d, pos, tk.TK_EXPAND_FP8_E4M3_1X128, cap)
    n_rows = offsets[hi - lo:]
    y = tk.tk_expert_standin(xq, sc, n_rows, 0.5)
    out = tk.tk_reduce(y, pos, w)
    torch.cuda.synchronize()

    # route + map: full, bit-exact
    o_idx, o_w = oracle.route(cfg["logits"], None, k, **r)
    assert np.array_equal(to_host(idx), o_idx)
    g_w = to_host(w)
    assert np.allclose(g_w, o_w, rtol=W_RTOL, atol=W_ATOL)
    oc, oo, op, ors = oracle.map_routes(o_idx, E, lo, hi)
    assert np.array_equal(to_host(counts), oc) and np.array_equal(to_host(offsets), oo)
    assert np.array_equal(to_host(pos), op)
    R = int(oo[-1])
    assert np.array_equal(to_host(row_src)[:R], ors)
    # the workload's structure: some local experts get no token, many tokens none
    assert (oc == 0).any(), "log-Zipf offset should leave some local experts empty"
    no_local = (op < 0).all(1)
    assert no_local.any() and (~no_local).any()

    # expand / stand-in / reduce: every row and every token, against the
    # oracle's own chain (the oracle's expand is given only the tokens with a
    # local route: the others write no row)
    act = ~no_local
    o_xq, o_sc = oracle.expand(cfg["x"][act], op[act], 1, R)
    g_xq, g_sc = to_host(xq[:R]), to_host(sc[:R])
    bad = np.nonzero((g_xq != o_xq).any(1))[0]
    assert bad.size == 0, f"FP8 rows differ: {bad.size} of {R}, first {bad[:4]}"
    assert np.array_equal(g_sc, o_sc)
    o_y = oracle.standin(o_xq, o_sc, 0.5)
    assert np.array_equal(to_host(y[:R]), o_y)
    g_out = to_host(out)
    rep = combine_report(g_out, oracle.reduce(o_y, op, o_w.astype(np.float32)))
    print(f"ep_share combine, all {T} tokens: {rep}")
    assert rep["ok"], rep
    assert np.all(g_out[no_local] == 0)


@pytest.mark.slow
def test_pipeline_v3_metric_shape():
    g = synth.v3_gate(0)
    T, E, k = g["T"], g["E"], g["k"]
    r = g["route"]
    x = synth.v3_hidden(0)
    H = x.shape[1]
    R = T * k
    idx, w = tk.tk_route(to_dev(g["logits"]), to_dev(g["bias"]), k, tk.RouteOpts(**r))
    counts, offsets, pos, row_src = tk.tk_map(idx, E)
    xq, sc = tk.tk_expand_quant(to_dev(x, bf16=True), pos, tk.TK_EXPAND_FP8_E4M3_1X128, R)
    torch.cuda.synchronize()
    g_xq, g_sc = to_host(xq), to_host(sc)
    del xq, sc
    y = synth.v3_expert_out(0, R, H)
    out = tk.tk_reduce_dense(to_dev(y, bf16=True), pos, w)
    torch.cuda.synchronize()

    o_idx, o_w = oracle.route(g["logits"], g["bias"], k, **r)
    assert np.array_equal(to_host(idx), o_idx)
    assert np.allclose(to_host(w), o_w, rtol=W_RTOL, atol=W_ATOL)
    oc, oo, op, ors = oracle.map_routes(o_idx, E)
    assert np.array_equal(to_host(counts), oc) and np.array_equal(to_host(offsets), oo)
    assert np.array_equal(to_host(pos), op) and np.array_equal(to_host(row_src), ors)
    o_xq, o_sc = oracle.expand(x, op, 1, R)
    bad = np.nonzero((g_xq != o_xq).any(1))[0]
    assert bad.size == 0, f"FP8 rows differ: {bad.size} of {R}, first {bad[:4]}"
    assert np.array_equal(g_sc, o_sc)
    rep = combine_report(to_host(out), oracle.reduce(y, op, o_w.astype(np.float32)))
    print(f"v3 metric-shape combine, all {T} tokens: {rep}")
    assert rep["ok"], rep
