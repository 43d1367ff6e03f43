"""GPU parity of tk_balance_loss against the CPU oracle.

f (a scaled integer count): within fp32 rounding of the oracle's fp64 value.
P and the loss: fp32 sums of T terms in a fixed order against fp64 sums;
each p is within a few ulp (pinned sigmoid, normalisation), and each fp32
addition adds at most 2^-24 relative to a partial sum, so 2e-5 relative
covers the deepest chain used here (4 + 8 + T/256 + 8 additions) with margin.
Determinism: bitwise equal over repeated calls, also when several final
workgroups race to be the one that forms the loss.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")

P_RTOL = 2e-5


def _check(logits, idx, score):
    f, P, loss = tk.tk_balance_loss(to_dev(logits), to_dev(idx), score)
    torch.cuda.synchronize()
    of, oP, oloss = oracle.balance_loss(logits, idx, score)
    assert np.allclose(to_host(f), of, rtol=1.2e-7, atol=0), "f"
    assert np.allclose(to_host(P), oP, rtol=P_RTOL, atol=0), np.max(np.abs(to_host(P) / oP - 1))
    assert abs(float(to_host(loss)[0]) - oloss) <= P_RTOL * abs(oloss)


@pytest.mark.parametrize("score", [tk.TK_SCORE_SIGMOID, tk.TK_SCORE_SOFTMAX])
@pytest.mark.parametrize("T,E,k", [(1, 8, 1), (33, 16, 2), (300, 100, 6), (513, 256, 8),
                                   (64, 1024, 32), (100, 5, 5), (4000, 64, 4),
                                   (70001, 256, 8)])   # 2188 tiles: many final-pass batches
def test_balance_random(T, E, k, score):
    rng = np.random.default_rng(T * 7 + E + k + score)
    logits = synth.normal_f32(rng, (T, E))
    idx, _ = oracle.route(logits, None, k, score)
    _check(logits, idx, score)


def test_balance_v3_full():
    cfg = synth.v3_gate(0)
    idx, _ = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    _check(cfg["logits"], idx, tk.TK_SCORE_SIGMOID)


def test_balance_closed_forms_and_determinism():
    rng = np.random.default_rng(91)
    T, E, k = 1024, 64, 4                          # T*k a multiple of E
    even = (np.arange(T * k) % E).reshape(T, k).astype(np.int32)
    eq = np.repeat(synth.normal_f32(rng, (T, 1)), E, axis=1)
    f, P, loss = (to_host(t) for t in tk.tk_balance_loss(to_dev(eq), to_dev(even),
                                                        tk.TK_SCORE_SIGMOID))
    assert np.all(f == 1.0)                        # even load: E/(kT) * kT/E
    assert np.allclose(P, 1.0 / E, rtol=1e-6)      # equal scores
    assert abs(loss[0] - 1.0) < 1e-5
    x = to_dev(synth.normal_f32(rng, (T, E)))
    idx = to_dev(synth.random_routing(rng, T, E, k))
    a = [to_host(t) for t in tk.tk_balance_loss(x, idx, tk.TK_SCORE_SIGMOID)]
    b = [to_host(t) for t in tk.tk_balance_loss(x, idx, tk.TK_SCORE_SIGMOID)]
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


def test_balance_deterministic_across_final_workgroups():
    """E = 256: eight final workgroups; whichever finishes last forms the loss
    from all of them, so five calls must agree bit for bit."""
    rng = np.random.default_rng(92)
    T, E, k = 8192, 256, 8
    x = to_dev(synth.normal_f32(rng, (T, E)))
    idx = to_dev(synth.random_routing(rng, T, E, k))
    runs = [[to_host(t) for t in tk.tk_balance_loss(x, idx, tk.TK_SCORE_SIGMOID)] for _ in range(5)]
    for r in runs[1:]:
        assert all(np.array_equal(u, v) for u, v in zip(runs[0], r))
