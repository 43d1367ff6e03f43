"""GPU parity of tk_route and tk_map against the CPU oracle.

Indices, counts, offsets, positions and row_src: bit-exact.  Weights: within
the fp32-vs-fp64 tolerance of tk_testutil (W_RTOL).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import W_ATOL, W_RTOL, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def _route_both(logits, bias, k, **r):
    opts = tk.RouteOpts(**r)
    idx, w = tk.tk_route(to_dev(logits), None if bias is None else to_dev(bias), k, opts)
    torch.cuda.synchronize()
    o_idx, o_w = oracle.route(logits, bias, k, **r)
    return to_host(idx), to_host(w), o_idx, o_w


def _assert_route(logits, bias, k, **r):
    g_idx, g_w, o_idx, o_w = _route_both(logits, bias, k, **r)
    bad = np.nonzero((g_idx != o_idx).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens differ, first t={bad[:5]}: {g_idx[bad[:2]]} vs {o_idx[bad[:2]]}"
    assert np.allclose(g_w, o_w, rtol=W_RTOL, atol=W_ATOL), np.abs(g_w - o_w).max()
    return g_idx, g_w


def test_route_tiny_softmax():
    cfg = synth.tiny(0)
    _assert_route(cfg["logits"], None, cfg["k"], **cfg["route"])


def test_route_v3_gate_full():
    cfg = synth.v3_gate(0)
    idx, w = _assert_route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    assert np.allclose(w.astype(np.float64).sum(1), 2.5, rtol=8 * 2.0 ** -24)


@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (3, 16, 4), (257, 64, 6), (130, 100, 7),
                                   (129, 128, 8), (200, 256, 8), (65, 512, 16),
                                   (33, 1024, 32), (50, 5, 5)])
@pytest.mark.parametrize("score", ["softmax", "sigmoid", "sigmoid_bias", "softmax_raw", "sigmoid_raw"])
def test_route_plain_shapes(T, E, k, score):
    rng = np.random.default_rng(T * 1000 + E + k)
    logits = synth.normal_f32(rng, (T, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32) if score == "sigmoid_bias" else None
    r = dict(score=tk.TK_SCORE_SOFTMAX if score.startswith("softmax") else tk.TK_SCORE_SIGMOID,
             n_groups=1, topk_groups=1, group_topn=0,
             renormalize=0 if score.endswith("raw") else 1, route_scale=1.5)
    _assert_route(logits, bias, k, **r)


@pytest.mark.parametrize("E,n_groups,topk_groups,group_topn,k", [
    (256, 8, 4, 2, 8), (64, 8, 3, 1, 5), (16, 4, 2, 2, 3), (128, 4, 2, 3, 6),
    (512, 8, 2, 2, 8), (1024, 16, 4, 2, 8), (256, 2, 1, 2, 4), (256, 4, 4, 2, 8),
    # group sizes spanning 1/4 lane .. 32 lanes, group_topn 1 and 2, k 3..8
    (64, 8, 3, 1, 4), (128, 4, 2, 2, 6), (128, 2, 1, 2, 8), (32, 16, 4, 2, 5),
    (64, 16, 8, 2, 3), (256, 64, 8, 2, 8), (256, 32, 4, 2, 8), (256, 16, 4, 1, 7),
])
def test_route_group_limited(E, n_groups, topk_groups, group_topn, k):
    rng = np.random.default_rng(E + n_groups * 10 + k)
    T = 333
    logits = synth.normal_f32(rng, (T, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    r = dict(score=tk.TK_SCORE_SIGMOID, n_groups=n_groups, topk_groups=topk_groups,
             group_topn=group_topn, renormalize=1, route_scale=2.5)
    _assert_route(logits, bias, k, **r)
    _assert_route(logits, None, k, **r)


# From T = 12288 on, 128 < E <= 256 takes the two-tokens-per-wave form (odd T
# leaves the last wave's second half without a token); every group layout it
# accepts, both score functions, with and without bias.
@pytest.mark.parametrize("T", [12288, 12289])
@pytest.mark.parametrize("E,n_groups,topk_groups,group_topn,k,score,with_bias", [
    (256, 8, 4, 2, 8, 1, True), (256, 8, 4, 2, 8, 1, False), (256, 1, 1, 0, 8, 0, False),
    (256, 1, 1, 0, 6, 1, True), (192, 3, 2, 2, 7, 1, True), (256, 16, 4, 1, 7, 1, True),
    (256, 32, 8, 2, 8, 1, False), (136, 1, 1, 0, 3, 0, False), (256, 2, 1, 2, 4, 1, True),
])
def test_route_two_tokens_per_wave(T, E, n_groups, topk_groups, group_topn, k, score, with_bias):
    rng = np.random.default_rng(T + E + 7 * n_groups + k)
    logits = synth.normal_f32(rng, (T, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32) if with_bias else None
    _assert_route(logits, bias, k, score=score, n_groups=n_groups, topk_groups=topk_groups,
                  group_topn=group_topn, renormalize=1, route_scale=2.5)


def test_route_two_tokens_per_wave_ties():
    # many equal keys and signed zeros at the large-T form's sizes
    rng = np.random.default_rng(9)
    x = rng.integers(-2, 3, (12289, 256)).astype(np.float32)
    x[rng.random(x.shape) < 0.2] = -0.0
    _assert_route(x, None, 8, score=1, n_groups=8, topk_groups=4, group_topn=2,
                  renormalize=1, route_scale=2.5)
    _assert_route(x, None, 8, score=0, n_groups=1, topk_groups=1, group_topn=0,
                  renormalize=1, route_scale=1.0)


def test_route_ties_and_signed_zero():
    rng = np.random.default_rng(5)
    for E, k in ((16, 4), (256, 8), (64, 32), (32, 32)):
        x = rng.integers(-3, 4, (300, E)).astype(np.float32)
        x[rng.random(x.shape) < 0.2] = -0.0
        _assert_route(x, None, k, score=0, n_groups=1, topk_groups=1, group_topn=0,
                      renormalize=1, route_scale=1.0)
        _assert_route(x, None, min(k, 8), score=1, n_groups=1, topk_groups=1, group_topn=0,
                      renormalize=1, route_scale=1.0)
    x = rng.integers(-2, 3, (300, 256)).astype(np.float32)
    _assert_route(x, None, 8, score=1, n_groups=8, topk_groups=4, group_topn=2,
                  renormalize=1, route_scale=2.5)


def test_route_extreme_logits():
    rng = np.random.default_rng(6)
    x = synth.normal_f32(rng, (200, 256)) * np.float32(40.0)   # sigmoid saturates to 0/1
    x[:, :3] = np.float32([-100.0, 100.0, 88.5])
    _assert_route(x, None, 8, score=1, n_groups=8, topk_groups=4, group_topn=2,
                  renormalize=1, route_scale=2.5)


def test_route_non_finite_logits_stay_in_range():
    # non-finite logits are outside the contract (experts and weights
    # unspecified, an expert may repeat), but every index is an expert id,
    # and the map still gives each routed slot (the first occurrence of an
    # id in its token) a distinct row: the routed positions are exactly
    # 0 .. R-1 and row_src[pos[t, j]] == t
    for T in (300, 12288):     # one token per wave; two per wave from T = 12288
        _non_finite_case(np.random.default_rng(16), T)


def _non_finite_case(rng, T):
    E, k = 256, 8
    x = synth.normal_f32(rng, (T, E))
    bad = rng.random((T, E)) < 0.05
    specials = np.array([np.nan, np.inf, -np.inf], np.float32)
    x[bad] = specials[rng.integers(0, 3, int(bad.sum()))]
    x[:4] = np.nan                                   # whole rows of NaN
    x.view(np.uint32)[4:8] = 0xFFFFFFFF              # NaN with every bit set
    x[8] = np.inf
    x[9] = -np.inf
    for score, groups in ((1, (8, 4, 2)), (0, (1, 1, 0)), (1, (1, 1, 0))):
        r = dict(score=score, n_groups=groups[0], topk_groups=groups[1], group_topn=groups[2],
                 renormalize=1, route_scale=2.5)
        idx, w = tk.tk_route(to_dev(x), None, k, tk.RouteOpts(**r))
        counts, offsets, pos, row_src = tk.tk_map(idx, E)
        torch.cuda.synchronize()
        g_idx, g_pos, g_rs = to_host(idx), to_host(pos), to_host(row_src)
        assert ((g_idx >= 0) & (g_idx < E)).all(), "an index outside [0, E)"
        R = int(to_host(offsets)[-1])
        routed = g_pos >= 0
        earlier = (g_idx[:, :, None] == g_idx[:, None, :]) & np.tri(k, k, -1, dtype=bool)[None]
        first = ~earlier.any(2)
        assert np.array_equal(routed, first)
        assert np.array_equal(np.sort(g_pos[routed]), np.arange(R))
        tok = np.repeat(np.arange(T), k).reshape(T, k)
        assert np.array_equal(g_rs[g_pos[routed]], tok[routed])


def test_route_zero_tokens():
    opts = tk.RouteOpts(score=1)
    idx, w = tk.tk_route(torch.empty((0, 64), device="cuda"), None, 4, opts)
    torch.cuda.synchronize()
    assert idx.shape == (0, 4)


# --------------------------------------------------------------------- map --
def _map_both(idx, E, lo, hi):
    g = tk.tk_map(to_dev(idx), E, lo, hi)
    torch.cuda.synchronize()
    counts, offsets, pos, row_src = (to_host(t) for t in g)
    o = oracle.map_routes(idx, E, lo, hi)
    return (counts, offsets, pos, row_src), o


def _assert_map(idx, E, lo, hi):
    (c, o, p, rs), (oc, oo, op, ors) = _map_both(idx, E, lo, hi)
    assert np.array_equal(c, oc), "counts"
    assert np.array_equal(o, oo), "offsets"
    bad = np.nonzero((p != op).any(1))[0]
    assert bad.size == 0, f"pos differs at tokens {bad[:5]}"
    R = int(oo[-1])
    assert np.array_equal(rs[:R], ors), "row_src"
    return c, o, p


def test_map_v3_gate_full():
    cfg = synth.v3_gate(0)
    r = cfg["route"]
    idx, _ = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **r)
    c, o, p = _assert_map(idx, 256, 0, 256)
    assert o[-1] == 8192 * 8


@pytest.mark.parametrize("T,E,k,lo,hi", [
    (1, 8, 1, 0, 8), (31, 16, 2, 0, 16), (1000, 256, 8, 32, 64), (4097, 256, 8, 0, 256),
    (777, 64, 3, 0, 64), (300, 1024, 32, 0, 1024), (512, 1024, 9, 100, 900),
    (2049, 32, 4, 7, 8), (5000, 160, 6, 0, 160), (70000, 256, 8, 0, 256),
    # count + place with the per-tile counts summed in place (small count
    # matrix: a masked range, or 64 experts) or scanned in a third launch
    # (more than 32768 counts), around 2^18 routes
    (32768, 256, 8, 0, 256), (32769, 256, 8, 0, 256), (40000, 256, 8, 32, 64),
    (33000, 64, 8, 0, 64),
    # one tile (the single-launch map): a full 256-token tile, a masked range,
    # 1024 experts (128-token tiles) with k = 32, the tiny softmax shape
    (256, 256, 8, 0, 256), (200, 64, 5, 10, 50), (128, 1024, 32, 0, 1024), (64, 16, 2, 0, 16),
])
def test_map_random_routing(T, E, k, lo, hi):
    rng = np.random.default_rng(T + E)
    idx = synth.random_routing(rng, T, E, k)
    _assert_map(idx, E, lo, hi)


@pytest.mark.parametrize("T", [600, 100, 40000])   # three tiles; one tile; two launches
def test_map_repeats_and_out_of_range_ids(T):
    rng = np.random.default_rng(7)
    E, k = 32, 6
    idx = rng.integers(-3, E + 3, (T, k)).astype(np.int32)   # repeats and invalid ids
    _assert_map(idx, E, 0, E)
    _assert_map(idx, E, 10, 20)


@pytest.mark.parametrize("T", [500, 100])   # two tiles; one tile
def test_map_empty_experts_and_all_masked(T):
    rng = np.random.default_rng(8)
    idx = synth.random_routing(rng, T, 16, 4) + 16            # all ids in [16, 32)
    (c, o, p, _), _ = _map_both(idx.astype(np.int32), 64, 0, 16)
    assert np.all(c == 0) and np.all(o == 0) and np.all(p == -1)


def test_map_zero_tokens():
    counts, offsets, pos, _ = tk.tk_map(torch.empty((0, 8), dtype=torch.int32, device="cuda"), 256)
    torch.cuda.synchronize()
    assert np.all(to_host(counts) == 0) and np.all(to_host(offsets) == 0)


def test_map_deterministic():
    rng = np.random.default_rng(9)
    idx = to_dev(synth.random_routing(rng, 8192, 256, 8))
    a = [to_host(t) for t in tk.tk_map(idx, 256)]
    b = [to_host(t) for t in tk.tk_map(idx, 256)]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


# ------------------------------------------------------------- aligned map --
@pytest.mark.parametrize("T,E,k,lo,hi,align", [
    (1, 8, 1, 0, 8, 128), (300, 16, 2, 0, 16, 1), (1000, 256, 8, 32, 64, 128),
    (4097, 256, 8, 0, 256, 128), (777, 64, 3, 0, 64, 7), (2049, 32, 4, 7, 8, 1000),
    (70000, 256, 8, 0, 256, 64), (300, 1024, 32, 0, 1024, 16),
    (200, 256, 8, 0, 256, 128), (100, 1024, 32, 0, 1024, 16), (64, 64, 4, 8, 40, 3),
    (40000, 64, 8, 0, 64, 128), (33000, 256, 8, 0, 256, 32),
])
def test_map_aligned_random_routing(T, E, k, lo, hi, align):
    rng = np.random.default_rng(T + E + align)
    idx = synth.random_routing(rng, T, E, k)
    g = [to_host(t) for t in tk.tk_map_aligned(to_dev(idx), E, lo, hi, align)]
    torch.cuda.synchronize()
    oc, oo, op, ors = oracle.map_aligned(idx, E, lo, hi, align)
    assert np.array_equal(g[0], oc), "counts"
    assert np.array_equal(g[1], oo), "offsets"
    assert np.array_equal(g[2], op), "pos"
    assert np.array_equal(g[3][: int(oo[-1])], ors), "row_src (with -1 on padding rows)"


def test_map_aligned_v3_full():
    cfg = synth.v3_gate(0)
    idx, _ = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    g = [to_host(t) for t in tk.tk_map_aligned(to_dev(idx), 256, 0, 256, 128)]
    oc, oo, op, ors = oracle.map_aligned(idx, 256, 0, 256, 128)
    assert np.array_equal(g[0], oc) and np.array_equal(g[1], oo) and np.array_equal(g[2], op)
    assert np.array_equal(g[3][: int(oo[-1])], ors)
    assert np.all(oo % 128 == 0)


def test_aligned_layout_gives_the_same_rows_and_combine():
    """Expanded rows and the combine do not depend on the layout: with y rows
    moved to the aligned positions, the reduce output is bitwise the same."""
    rng = np.random.default_rng(90)
    T, E, k, H, align = 700, 32, 4, 1024, 128
    idx = synth.random_routing(rng, T, E, k)
    x = synth.normal_bf16(rng, (T, H))
    w = rng.random((T, k)).astype(np.float32)
    idx_d, x_d, w_d = to_dev(idx), to_dev(x, bf16=True), to_dev(w)
    _, off_p, pos_p, _ = tk.tk_map(idx_d, E)
    _, off_a, pos_a, _ = tk.tk_map_aligned(idx_d, E, 0, E, align)
    R, cap = T * k, T * k + E * (align - 1)
    assert int(off_a[-1]) <= cap
    xq_p, sc_p = tk.tk_expand_quant(x_d, pos_p, tk.TK_EXPAND_FP8_E4M3_1X128, R)
    xq_a, sc_a = tk.tk_expand_quant(x_d, pos_a, tk.TK_EXPAND_FP8_E4M3_1X128, cap)
    pp, pa = pos_p.view(-1).long(), pos_a.view(-1).long()
    assert torch.equal(xq_a[pa], xq_p[pp]) and torch.equal(sc_a[pa], sc_p[pp])
    y_p = to_dev(synth.normal_bf16(rng, (R, H)), bf16=True)
    y_a = torch.zeros((cap, H), dtype=torch.bfloat16, device="cuda")
    y_a[pa] = y_p[pp]
    out_p = tk.tk_reduce(y_p, pos_p, w_d)
    out_a = tk.tk_reduce(y_a, pos_a, w_d)
    torch.cuda.synchronize()
    assert torch.equal(out_p.view(torch.int16), out_a.view(torch.int16))
