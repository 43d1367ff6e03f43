"""A seeded sweep of the whole routing path over mixed configurations, each
step against the oracle: route (softmax or sigmoid, with or without bias,
group limiting, renormalisation, scaling), the map with a random local range
and segment alignment, the expand (FP8 or bf16, sometimes with a capacity
below the row count) and the reduce.  Shapes are small and ragged: T from 1
to 700 tokens, E from 8 to 512 experts, k up to 8, H from 128 to 7168.

Bars as in the per-step tests: indices, counts, offsets, positions, row
sources, bf16 rows, FP8 codes and scales bit-exact; weights within 4e-6
relative; the combine within 1e-2 + 1e-2 |ref|.
"""
import numpy as np
import pytest

import oracle
from moe_routing_amd import synth
from tk_testutil import W_ATOL, W_RTOL, combine_report, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")

# (E, n_groups, topk_groups, group_topn) with power-of-two lane runs per group
GROUPED = [(256, 8, 4, 2), (128, 8, 4, 2), (64, 4, 2, 2), (256, 8, 3, 1)]


def _routing(rng):
    if rng.random() < 0.5:
        E, ng, tg, gt = GROUPED[int(rng.integers(len(GROUPED)))]
        score = tk.TK_SCORE_SIGMOID
    else:
        E = int(rng.choice([8, 16, 32, 64, 100, 128, 256, 512]))
        ng, tg, gt = 1, 1, 0
        score = int(rng.choice([tk.TK_SCORE_SOFTMAX, tk.TK_SCORE_SIGMOID]))
    k = int(rng.integers(1, min(E, 8) + 1))
    r = dict(score=score, n_groups=ng, topk_groups=tg, group_topn=gt,
             renormalize=int(rng.integers(0, 2)), route_scale=float(rng.choice([1.0, 2.5])))
    bias = None
    if score == tk.TK_SCORE_SIGMOID and rng.random() < 0.5:
        bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return E, k, r, bias


@pytest.mark.parametrize("seed", range(48))
def test_path_sweep(seed):
    rng = np.random.default_rng(5000 + seed)
    E, k, r, bias = _routing(rng)
    T = int(rng.integers(1, 701))
    H = int(rng.choice([128, 256, 384, 1152, 7168]))
    logits = synth.normal_f32(rng, (T, E))

    idx, w = tk.tk_route(to_dev(logits), None if bias is None else to_dev(bias), k,
                         tk.RouteOpts(**r))
    o_idx, o_w = oracle.route(logits, bias, k, **r)
    assert np.array_equal(to_host(idx), o_idx), (E, k, r)
    assert np.allclose(to_host(w), o_w, rtol=W_RTOL, atol=W_ATOL), (E, k, r)

    lo = int(rng.integers(0, E))
    hi = int(rng.integers(lo + 1, E + 1))
    align = int(rng.choice([1, 1, 8, 128]))
    counts, offsets, pos, row_src = tk.tk_map_aligned(idx, E, lo, hi, align)
    oc, oo, op, ors = oracle.map_aligned(o_idx, E, lo, hi, align)
    n = int(oo[-1])
    assert np.array_equal(to_host(counts), oc) and np.array_equal(to_host(offsets), oo)
    assert np.array_equal(to_host(pos), op)
    assert np.array_equal(to_host(row_src)[:n], ors[:n])

    x = synth.normal_bf16(rng, (T, H))
    cap = max(n if rng.random() < 0.8 else n // 2, 1)
    mode = int(rng.choice([tk.TK_EXPAND_FP8_E4M3_1X128, tk.TK_EXPAND_BF16]))
    out, sc = tk.tk_expand_quant(to_dev(x, bf16=True), pos, mode, cap)
    o_out, o_sc = oracle.expand(x, op, mode, cap)
    rows = np.unique(op[(op >= 0) & (op < cap)])
    assert np.array_equal(to_host(out)[rows], o_out[rows])
    if mode == tk.TK_EXPAND_FP8_E4M3_1X128:
        assert np.array_equal(to_host(sc)[rows], o_sc[rows])

    y = synth.normal_bf16(rng, (max(n, 1), H))
    got = tk.tk_reduce(to_dev(y, bf16=True), pos, w)
    rep = combine_report(to_host(got), oracle.reduce(y, op, o_w.astype(np.float32)))
    assert rep["ok"], rep


# tk_reduce_dense around its thresholds: rows of H = 1536 (the one-wave-per-unit
# kernel) and longer (the staged form), partly filled 512-column units, every
# compiled k, T from just below to a few rounds above (compute units) x 16
# tokens, and k = 8 with H = 7168 (one launch per round).  Positions are a
# routing from the oracle's map of random expert choices (expert-contiguous
# rows, as tk_map lays them out), with a few slots masked; y is drawn on the
# device.  The dense combine must equal tk_reduce bit for bit on every token,
# and sampled tokens (first, last, random) are compared with the oracle.
DENSE_H = [1536, 1544, 2048, 2056, 2568, 3072, 4096, 5120, 6144, 7168]


@pytest.mark.parametrize("seed", range(24))
def test_reduce_dense_sweep(seed):
    import torch
    rng = np.random.default_rng(1000 + seed)
    k = int(rng.choice([1, 2, 4, 6, 8]))
    H = 7168 if seed % 4 == 0 else int(rng.choice(DENSE_H))
    if seed % 4 == 0:
        k = 8
    E = 256
    T_max = max(4200, min(16000, (300 << 20) // (k * H)))
    T = int(rng.integers(3800, T_max + 1))
    R = T * k
    idx = synth.random_routing(rng, T, E, k)
    _, _, pos, _ = oracle.map_routes(idx, E)
    pos = pos.copy()
    pos[rng.random((T, k)) < 0.05] = -1
    w = rng.uniform(0.05, 0.6, (T, k)).astype(np.float32)
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    y = torch.randn((R, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    pd, wd = to_dev(pos), to_dev(w)
    dense = tk.tk_reduce_dense(y, pd, wd)
    plain = tk.tk_reduce(y, pd, wd)
    torch.cuda.synchronize()
    print(f"dense sweep seed {seed}: T={T} k={k} H={H}", flush=True)
    assert torch.equal(dense, plain), "tk_reduce_dense differs from tk_reduce"
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 40, replace=False)]))
    rows = pos[sample]
    used = rows[rows >= 0]
    y_s = to_host(y[torch.from_numpy(used.astype(np.int64)).to(dev)])
    # the sampled tokens' rows renumbered 0.. in order, masked slots kept masked
    pos_s = np.full(rows.shape, -1, np.int32)
    pos_s[rows >= 0] = np.arange(used.size, dtype=np.int32)
    rep = combine_report(to_host(dense[torch.from_numpy(sample).to(dev)]),
                         oracle.reduce(y_s, pos_s, w[sample]))
    assert rep["ok"], rep
