"""End-to-end GPU pipelines against the CPU oracle: each step's GPU output
feeds the next GPU step, and every stage is compared with the oracle run on
the same inputs.

tiny      T=64, E=16, k=2, H=256: softmax top-2, bf16 expand, reduce.
ep_share  T=32768, H=7168, E=256, k=8, one expert-parallel rank's share
          (experts 32..63 local), v3 gating with a log-Zipf popularity offset:
          route, map with the local mask, FP8 expand, stand-in expert
          (dequantise * 0.5), reduce -- all full size on the GPU; the oracle
          checks route and map in full and expand / stand-in / reduce on a
          sample of tokens.
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

    # expand / stand-in / reduce: a sample of tokens with and without local routes
    rng = np.random.default_rng(40)
    sample = np.concatenate([rng.choice(np.nonzero(~no_local)[0], 96, replace=False),
                             rng.choice(np.nonzero(no_local)[0], 32, replace=False)])
    xs = cfg["x"][sample]
    q_ref, s_ref = oracle.quant_row(xs)
    rows = np.array(sorted({int(p) for p in op[sample].ravel() if p >= 0}), np.int64)
    ridx = torch.from_numpy(rows).to(xq.device)
    g_q, g_s, g_y = (to_host(t.index_select(0, ridx)) for t in (xq, sc, y))
    where = {int(r): i for i, r in enumerate(rows)}
    for i, t in enumerate(sample):
        for j in range(k):
            p = op[t, j]
            if p >= 0:
                assert np.array_equal(g_q[where[p]], q_ref[i]) and np.array_equal(g_s[where[p]], s_ref[i])
    # stand-in reference from the oracle's own codes: row -> token -> q_ref
    i_of_t = {int(t): i for i, t in enumerate(sample)}
    src = np.array([i_of_t[int(ors[r])] for r in rows])
    y_ref = oracle.standin(q_ref[src], s_ref[src], 0.5)
    assert np.array_equal(g_y, y_ref)
    # reduce over the oracle's own stand-in rows, positions renumbered to them
    pos_s = np.vectorize(lambda p: where.get(int(p), -1))(op[sample]).astype(np.int32)
    ref = oracle.reduce(y_ref, pos_s, o_w[sample].astype(np.float32))
    g_out = to_host(out.index_select(0, torch.from_numpy(sample).to(out.device)))
    rep = combine_report(g_out, ref)
    assert rep["ok"], rep
    assert np.all(g_out[no_local[sample]] == 0)
