"""Pins of the oracle's expand (bf16 copy, 1x128 FP8 quantisation), stand-in
expert and reduce (combine).

FP8: scales against torch fp32 amax/448, codes against torch's float8 cast of
torch's fp32 quotient, plus the block-scale invariants (every unclamped block
holds a +-448 code; round-trip error bounded by the block scale).
Reduce: against an fp64 torch sum (the result must be the bf16 value nearest
to it) and closed forms (k=1, w=1 is an exact gather; no valid route gives 0).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth


def _f32(bits16):
    return (np.asarray(bits16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _torch_quant(x_bits: np.ndarray):
    x = torch.from_numpy(_f32(x_bits))                      # (n, H) fp32, exact
    n, H = x.shape
    xb = x.view(n, H // 128, 128)
    amax = xb.abs().amax(dim=2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    scale = amax / torch.tensor(448.0, dtype=torch.float32)    # IEEE fp32 division
    q = (xb / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(n, H).numpy(), scale.numpy()


def _special_rows(H):
    rows = []
    rows.append(np.zeros(H, np.float32))                    # clamp: amax < 1e-4
    z = np.full(H, -0.0, np.float32); rows.append(z)          # signed zeros
    t = np.full(H, 3e-5, np.float32); t[::2] *= -1; rows.append(t)   # tiny, clamped
    g = np.linspace(-448, 448, H).astype(np.float32); rows.append(g)  # scale 1 region
    rows.append(np.linspace(-1e4, 1e4, H).astype(np.float32))
    return synth.bf16_bits(np.stack(rows))


@pytest.mark.parametrize("H", [128, 256, 1024, 7168])
def test_quant_matches_torch_and_invariants(H):
    rng = np.random.default_rng(H)
    x = synth.normal_bf16(rng, (64, H))
    x[5] = synth.bf16_bits(synth.normal_f32(rng, (H,)) * np.float32(50.0))
    x = np.concatenate([x, _special_rows(H)])
    q, sc = oracle.quant_row(x)
    q2, sc2 = _torch_quant(x)
    assert np.array_equal(sc, sc2)
    assert np.array_equal(q, q2)
    xf = _f32(x).astype(np.float64)
    deq = oracle.e4m3_to_f64(q) * np.repeat(sc.astype(np.float64), 128, axis=1)
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.repeat(sc.astype(np.float64), 128, 1) * 2.0 ** -10)
    assert np.all(np.abs(xf - deq) <= bound * (1 + 2.0 ** -20))
    amax = np.abs(xf).reshape(x.shape[0], -1, 128).max(2)
    unclamped = amax >= 1e-4
    has448 = ((q.reshape(x.shape[0], -1, 128) & 0x7F) == 0x7E).any(2)
    assert np.all(has448[unclamped])
    assert np.all(sc[~unclamped] == np.float32(1e-4) / np.float32(448.0))


def test_expand_fp8_copies_and_skips():
    rng = np.random.default_rng(30)
    T, E, k, H = 50, 16, 3, 256
    idx = synth.random_routing(rng, T, E, k)
    _, offsets, pos, _ = oracle.map_routes(idx, E, 4, 12)
    R = int(offsets[-1])
    x = synth.normal_bf16(rng, (T, H))
    cap = R - 2                               # last two rows beyond capacity
    out, scales = oracle.expand(x, pos, 1, cap)
    q, sc = oracle.quant_row(x)
    written = np.zeros(cap, bool)
    for t in range(T):
        for j in range(k):
            r = pos[t, j]
            if 0 <= r < cap:
                assert np.array_equal(out[r], q[t]) and np.array_equal(scales[r], sc[t])
                written[r] = True
    assert written.all()
    outb, _ = oracle.expand(x, pos, 0, R)
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                assert np.array_equal(outb[pos[t, j]], x[t])


def test_standin_matches_torch():
    rng = np.random.default_rng(31)
    x = synth.normal_bf16(rng, (20, 512))
    q, sc = oracle.quant_row(x)
    y = oracle.standin(q, sc, 0.5)
    d = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float32)
    v = d * torch.from_numpy(np.repeat(sc, 128, axis=1))
    ref = (v * torch.tensor(0.5)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, ref)


def _bf16_nearest_ok(out_bits, ref64):
    """out must be a nearest bf16 value to ref64 (within half a bf16 ulp)."""
    out = _f32(out_bits).astype(np.float64)
    a = np.abs(ref64)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    half_ulp = 2.0 ** (e - 8)
    return np.all(np.abs(out - ref64) <= half_ulp)


@pytest.mark.parametrize("T,k,H", [(64, 2, 256), (300, 8, 512), (33, 1, 128)])
def test_reduce_is_rounded_fp64_sum(T, k, H):
    rng = np.random.default_rng(T * k)
    E = 16
    idx = synth.random_routing(rng, T, E, k)
    _, offsets, pos, _ = oracle.map_routes(idx, E, 0, E)
    R = int(offsets[-1])
    y = synth.normal_bf16(rng, (R, H))
    w = rng.random((T, k)).astype(np.float32)
    out = oracle.reduce(y, pos, w)
    yt = torch.from_numpy(_f32(y).astype(np.float64))
    g = yt[torch.from_numpy(pos.astype(np.int64))]          # (T, k, H)
    ref = (torch.from_numpy(w.astype(np.float64))[:, :, None] * g).sum(1).numpy()
    assert _bf16_nearest_ok(out, ref)
    assert np.array_equal(out, oracle.bf16_from_f64(ref))


def test_reduce_closed_forms():
    rng = np.random.default_rng(32)
    T, H = 40, 256
    y = synth.normal_bf16(rng, (T, H))
    perm = rng.permutation(T).astype(np.int32)
    # k = 1, w = 1: an exact gather
    out = oracle.reduce(y, perm[:, None], np.ones((T, 1), np.float32))
    assert np.array_equal(out, y[perm])
    # no valid route: +0
    pos = np.full((T, 3), -1, np.int32)
    out = oracle.reduce(y, pos, np.ones((T, 3), np.float32))
    assert np.all(out == 0)
    # masked slots do not contribute; weights of w=0.5 on two equal rows = the row
    pos = np.stack([perm, np.full(T, -1, np.int32), perm], 1)
    w = np.full((T, 3), 0.5, np.float32)
    out = oracle.reduce(y, pos, w)
    assert np.array_equal(out, y[perm])
