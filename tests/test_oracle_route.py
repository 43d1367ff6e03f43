"""Pins of the oracle's route step (score, group limit, top-k, weights).

Selection is checked by brute force: torch's stable descending sort of the
oracle's fp32 keys (a library routine), enumeration of group subsets, and a
hand-worked fixture of the listing's tie rule.  Weights are checked against
their invariants (sum = route_scale) and torch fp64 softmax / sigmoid.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _stable_topk(keys: np.ndarray, k: int, allowed: np.ndarray | None = None) -> np.ndarray:
    kt = torch.from_numpy(keys.astype(np.float64))
    if allowed is not None:
        kt = torch.where(torch.from_numpy(allowed), kt, torch.tensor(-np.inf, dtype=torch.float64))
    order = torch.sort(kt, dim=1, descending=True, stable=True).indices
    return order[:, :k].numpy().astype(np.int32)


def _ties_logits(rng, T, E):
    # small integer logits: many exact ties, including +0/-0
    x = rng.integers(-3, 4, (T, E)).astype(np.float32)
    x[rng.random((T, E)) < 0.1] = -0.0
    return x


@pytest.mark.parametrize("E,k", [(8, 1), (8, 3), (16, 2), (16, 4), (32, 8), (64, 6)])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_plain_topk_matches_stable_sort(E, k, kind):
    rng = np.random.default_rng(10 + E + k)
    T = 300
    x = synth.normal_f32(rng, (T, E)) if kind == "normal" else _ties_logits(rng, T, E)
    for score, bias in ((oracle.SOFTMAX, None), (oracle.SIGMOID, None),
                        (oracle.SIGMOID, rng.uniform(-0.1, 0.1, E).astype(np.float32))):
        idx, _ = oracle.route(x, bias, k, score)
        keys = oracle.route_keys(x, score, bias)
        assert np.array_equal(idx, _stable_topk(keys, k))


def test_golden_listing_tie_rule():
    """Hand-worked rows: k rounds of max with the lowest index winning ties."""
    with open(os.path.join(GOLDEN, "topk_listing_ties.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        x = np.array([c["logits"]], np.float32)
        idx, _ = oracle.route(x, None, c["k"], oracle.SOFTMAX)
        assert idx[0].tolist() == c["topk_idx"], c


def _group_reference(keys, n_groups, topk_groups, group_topn, k):
    T, E = keys.shape
    gs = E // n_groups
    kg = torch.from_numpy(keys).view(T, n_groups, gs)
    top = torch.sort(kg, dim=2, descending=True, stable=True).values[:, :, :group_topn]
    g = top[:, :, 0].clone()
    for i in range(1, group_topn):
        g = g + top[:, :, i]                        # fp32, largest first
    gorder = torch.sort(g, dim=1, descending=True, stable=True).indices[:, :topk_groups]
    gmask = torch.zeros(T, n_groups, dtype=torch.bool)
    gmask.scatter_(1, gorder, True)
    allowed = gmask.repeat_interleave(gs, dim=1).numpy()
    return _stable_topk(keys, k, allowed), g.numpy(), gmask.numpy()


@pytest.mark.parametrize("E,n_groups,topk_groups,group_topn,k", [
    (16, 4, 2, 2, 3), (32, 8, 4, 2, 8), (64, 8, 3, 1, 5), (256, 8, 4, 2, 8), (24, 3, 1, 3, 4),
])
@pytest.mark.parametrize("kind", ["normal", "ties"])
def test_group_limited_topk_brute_force(E, n_groups, topk_groups, group_topn, k, kind):
    rng = np.random.default_rng(E * 7 + k)
    T = 200
    x = synth.normal_f32(rng, (T, E)) if kind == "normal" else _ties_logits(rng, T, E)
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, _ = oracle.route(x, bias, k, oracle.SIGMOID, n_groups, topk_groups, group_topn)
    keys = oracle.route_keys(x, oracle.SIGMOID, bias)
    ref, g, gmask = _group_reference(keys, n_groups, topk_groups, group_topn, k)
    assert np.array_equal(idx, ref)
    # enumeration: the kept set of groups is a subset with the largest scores,
    # and among equally scored choices the lexicographically lowest
    for t in range(0, T, 17):
        best = None
        for sub in itertools.combinations(range(n_groups), topk_groups):
            key = (sorted((-float(g[t, s]) for s in sub)), sub)
            best = key if best is None or key < best else best
        assert sorted(np.nonzero(gmask[t])[0].tolist()) == list(best[1])


def test_group_limit_reduces_to_plain_topk():
    rng = np.random.default_rng(11)
    x = synth.normal_f32(rng, (500, 64))
    plain, _ = oracle.route(x, None, 6, oracle.SIGMOID)
    one, _ = oracle.route(x, None, 6, oracle.SIGMOID, 1, 1, 0)
    all_groups, _ = oracle.route(x, None, 6, oracle.SIGMOID, 8, 8, 2)
    assert np.array_equal(plain, one) and np.array_equal(plain, all_groups)


def test_weights_sigmoid_and_softmax():
    rng = np.random.default_rng(12)
    x = synth.normal_f32(rng, (400, 32))
    xt = torch.from_numpy(x.astype(np.float64))
    # sigmoid, renormalised, scale 2.5
    idx, w = oracle.route(x, None, 8, oracle.SIGMOID, route_scale=2.5)
    s = torch.sigmoid(torch.gather(xt, 1, torch.from_numpy(idx).long()))
    ref = (s / s.sum(1, keepdim=True) * 2.5).numpy()
    assert np.allclose(w, ref, rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 2.5, rtol=1e-14)
    # sigmoid, not renormalised
    _, w = oracle.route(x, None, 8, oracle.SIGMOID, renormalize=0, route_scale=1.5)
    assert np.allclose(w, s.numpy() * 1.5, rtol=1e-13)
    # softmax restricted to the chosen experts (renormalised top-k)
    idx, w = oracle.route(x, None, 4, oracle.SOFTMAX)
    ref = torch.softmax(torch.gather(xt, 1, torch.from_numpy(idx).long()), 1).numpy()
    assert np.allclose(w, ref, rtol=1e-13)
    assert np.allclose(w.sum(1), 1.0, rtol=1e-14)
    # also equal to: full softmax, take top-k entries, renormalise
    p = torch.softmax(xt, 1)
    pk = torch.gather(p, 1, torch.from_numpy(idx).long())
    assert np.allclose(w, (pk / pk.sum(1, keepdim=True)).numpy(), rtol=1e-12)
    # softmax over all experts, not renormalised
    _, w = oracle.route(x, None, 4, oracle.SOFTMAX, renormalize=0, route_scale=2.0)
    assert np.allclose(w, (pk * 2.0).numpy(), rtol=1e-12)


def test_softmax_shift_invariance():
    """softmax(x + c) = softmax(x): with logits on a 1/64 grid the shift by 4 is
    exact in fp32, so indices must be identical and weights equal."""
    rng = np.random.default_rng(13)
    x = (np.round(synth.normal_f32(rng, (300, 16)) * 64) / 64).astype(np.float32)
    xs = x + np.float32(4.0)
    assert np.array_equal(xs.astype(np.float64), x.astype(np.float64) + 4.0)
    i1, w1 = oracle.route(x, None, 2, oracle.SOFTMAX)
    i2, w2 = oracle.route(xs, None, 2, oracle.SOFTMAX)
    assert np.array_equal(i1, i2)
    assert np.allclose(w1, w2, rtol=1e-14)


def test_v3_gate_invariants():
    cfg = synth.v3_gate(0)
    r = cfg["route"]
    idx, w = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], r["score"], r["n_groups"],
                          r["topk_groups"], r["group_topn"], r["renormalize"], r["route_scale"])
    T, k = idx.shape
    assert (T, k) == (8192, 8)
    assert np.all((idx >= 0) & (idx < 256))
    assert all(len(set(row)) == k for row in idx.tolist())
    # at most 4 groups of 32 touched per token
    assert np.max([len(set((row // 32).tolist())) for row in idx]) <= 4
    assert np.allclose(w.sum(1), 2.5, rtol=1e-14)
    assert np.all(w > 0)
    # slot 0 has the largest biased key of the token
    keys = oracle.route_keys(cfg["logits"], r["score"], cfg["bias"])
    sel = np.take_along_axis(keys, idx.astype(np.int64), 1)
    assert np.all(np.diff(sel, axis=1) <= 0)
