"""Pins of the oracle's load-balance statistics and loss.

Against an fp64 torch evaluation (torch.sigmoid / torch.softmax, bincount),
closed forms (equal scores give P = 1/E and a loss of exactly 1 whatever the
routing; an even routing gives f = 1), and the bound loss <= E/k * max P.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth


def _torch_balance(logits, idx, score):
    x = torch.from_numpy(logits.astype(np.float64))
    T, E = x.shape
    k = idx.shape[1]
    if score == oracle.SIGMOID:
        s = torch.sigmoid(x)
        p = s / s.sum(1, keepdim=True)
    else:
        p = torch.softmax(x, 1)
    P = p.mean(0)
    count = torch.bincount(torch.from_numpy(idx.reshape(-1).astype(np.int64)), minlength=E)
    f = E / (k * T) * count.double()
    return f.numpy(), P.numpy(), float((f * P).sum())


@pytest.mark.parametrize("score", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("T,E,k", [(1, 8, 2), (300, 64, 6), (2048, 256, 8)])
def test_balance_matches_torch(T, E, k, score):
    rng = np.random.default_rng(T + E + score)
    logits = synth.normal_f32(rng, (T, E))
    idx, _ = oracle.route(logits, None, k, score)
    f, P, loss = oracle.balance_loss(logits, idx, score)
    f2, P2, loss2 = _torch_balance(logits, idx, score)
    assert np.array_equal(f, f2)                          # integer counts, exact scaling
    # sigmoid: the pinned fp32 scores are within 3 ulp of fp64
    tol = 8 * 2.0 ** -24 if score == oracle.SIGMOID else 1e-12
    assert np.allclose(P, P2, rtol=tol, atol=0)
    assert abs(loss - loss2) <= tol * abs(loss2)


@pytest.mark.parametrize("score", [oracle.SIGMOID, oracle.SOFTMAX])
def test_balance_closed_forms(score):
    rng = np.random.default_rng(5)
    T, E, k = 256, 32, 4
    # equal scores within each token: P = 1/E exactly, loss = 1 for any routing
    logits = np.repeat(synth.normal_f32(rng, (T, 1)), E, axis=1)
    idx = synth.random_routing(rng, T, E, k)
    f, P, loss = oracle.balance_loss(logits, idx, score)
    assert np.allclose(P, 1.0 / E, rtol=1e-14)
    assert abs(loss - 1.0) < 1e-12
    # a perfectly even routing (each expert chosen T*k/E times): f = 1
    even = (np.arange(T * k) % E).reshape(T, k).astype(np.int32)
    f, P, loss = oracle.balance_loss(synth.normal_f32(rng, (T, E)), even, score)
    assert np.all(f == 1.0)
    assert abs(loss - 1.0) < 1e-12                        # sum of P over experts is 1
    # everything on one expert: f = E/k there, loss = E/k * P_e
    one = np.zeros((T, k), np.int32)
    x = synth.normal_f32(rng, (T, E))
    f, P, loss = oracle.balance_loss(x, one, score)
    assert f[0] == E and np.all(f[1:] == 0)
    assert abs(loss - E * P[0]) < 1e-12
