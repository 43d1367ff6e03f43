"""Pins of the oracle's fused SwiGLU + per-token 1x128 FP8 quantisation.

The activation a = RN(RN(g * sigmoid(g)) * u) [* w] is checked against an
fp64 torch evaluation (error bound from the pinned sigmoid's 3 ulp and the
roundings) and against closed forms where the pinned sigmoid is exactly 1, 0
or 1/2.  The fp32 1x128 codec is checked against torch's fp32 amax/448 and
float8_e4m3fn cast on arbitrary fp32 rows, and by the block-scale invariants.
The row-weight scatter is checked against a brute-force inverse of pos.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth


def _f32(bits16):
    return (np.asarray(bits16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rows(rng, R, I, scale=2.0):
    g = synth.normal_f32(rng, (R, I)) * np.float32(scale)
    u = synth.normal_f32(rng, (R, I))
    return synth.bf16_bits(np.concatenate([g, u], axis=1))


def _torch_silu_mul64(h, I, row_w=None):
    x = torch.from_numpy(_f32(h).astype(np.float64))
    g, u = x[:, :I], x[:, I:]
    a = g * torch.sigmoid(g) * u
    if row_w is not None:
        a = a * torch.from_numpy(row_w.astype(np.float64))[:, None]
    return a.numpy()


@pytest.mark.parametrize("weighted", [False, True])
def test_swiglu_activation_vs_fp64(weighted):
    rng = np.random.default_rng(70 + weighted)
    R, I = 64, 512
    h = _rows(rng, R, I)
    rw = rng.uniform(0.01, 2.5, R).astype(np.float32) if weighted else None
    a = oracle.swiglu_f32(h, I, rw).astype(np.float64)
    ref = _torch_silu_mul64(h, I, rw)
    # sigmoid <= 3 ulp (pinned, measured 2.47), then 2 or 3 roundings
    bound = 7 * 2.0 ** -24 * np.abs(ref) + 1e-44
    assert np.all(np.abs(a - ref) <= bound), np.max(np.abs(a - ref) / np.maximum(np.abs(ref), 1e-30))


def test_swiglu_closed_forms():
    rng = np.random.default_rng(71)
    I = 256
    # g >= 20: the pinned sigmoid is exactly 1, so a = RN(g * u) (one rounding)
    g = rng.uniform(20.0, 80.0, (8, I)).astype(np.float32)
    u = synth.normal_f32(rng, (8, I))
    h = synth.bf16_bits(np.concatenate([g, u], 1))
    gb, ub = _f32(h[:, :I]), _f32(h[:, I:])
    assert np.array_equal(oracle.swiglu_f32(h, I), (gb * ub).astype(np.float32))
    w = np.float32(0.3)
    a_w = oracle.swiglu_f32(h, I, np.full(8, w, np.float32))
    assert np.array_equal(a_w, ((gb * ub).astype(np.float32) * w).astype(np.float32))
    # g <= -100: sigmoid is exactly 0, so a is a zero
    h2 = synth.bf16_bits(np.concatenate([np.full((2, I), -120.0, np.float32), u[:2]], 1))
    assert np.all(oracle.swiglu_f32(h2, I) == 0)
    # g = 0 (sigmoid 1/2) or u = 0: a is a zero; their codes are zeros
    h3 = synth.bf16_bits(np.concatenate([np.zeros((2, I), np.float32), u[:2]], 1))
    h4 = synth.bf16_bits(np.concatenate([g[:2], np.zeros((2, I), np.float32)], 1))
    for hz in (h3, h4):
        assert np.all(oracle.swiglu_f32(hz, I) == 0)
        q, sc = oracle.swiglu_quant(hz, I)
        assert np.all((q & 0x7F) == 0)
        assert np.all(sc == np.float32(1e-4) / np.float32(448.0))


def _torch_quant_f32(a):
    x = torch.from_numpy(np.ascontiguousarray(a, np.float32))
    n, H = x.shape
    xb = x.view(n, H // 128, 128)
    amax = xb.abs().amax(dim=2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    scale = amax / torch.tensor(448.0, dtype=torch.float32)
    q = (xb / scale[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8)
    return q.reshape(n, H).numpy(), scale.numpy()


def test_quant_f32_row_matches_torch():
    rng = np.random.default_rng(72)
    a = np.concatenate([
        synth.normal_f32(rng, (32, 1024)),
        synth.normal_f32(rng, (4, 1024)) * np.float32(1e-6),       # clamped blocks
        synth.normal_f32(rng, (4, 1024)) * np.float32(3e4),
        rng.uniform(-1, 1, (4, 1024)).astype(np.float32) ** 9,     # wide dynamic range
        np.full((1, 1024), -0.0, np.float32),
    ])
    q, sc = oracle.quant_f32_row(a)
    q2, sc2 = _torch_quant_f32(a)
    assert np.array_equal(sc, sc2)
    assert np.array_equal(q, q2)


@pytest.mark.parametrize("weighted", [False, True])
def test_swiglu_quant_invariants(weighted):
    rng = np.random.default_rng(73 + weighted)
    R, I = 48, 1024
    h = _rows(rng, R, I, scale=3.0)
    rw = rng.uniform(0.05, 2.5, R).astype(np.float32) if weighted else None
    q, sc = oracle.swiglu_quant(h, I, rw)
    a64 = _torch_silu_mul64(h, I, rw)
    scr = np.repeat(sc.astype(np.float64), 128, axis=1)
    deq = oracle.e4m3_to_f64(q) * scr
    # block-scale bound on the fp32 activations, plus their distance to fp64
    bound = np.maximum(np.abs(a64) * 2.0 ** -4, scr * 2.0 ** -10) * (1 + 2.0 ** -20) \
        + 8 * 2.0 ** -24 * np.abs(a64)
    assert np.all(np.abs(a64 - deq) <= bound)
    amax = np.abs(oracle.swiglu_f32(h, I, rw)).reshape(R, -1, 128).max(2)
    unclamped = amax >= 1e-4
    has448 = ((q.reshape(R, -1, 128) & 0x7F) == 0x7E).any(2)
    assert np.all(has448[unclamped])


def test_row_weights_inverse_of_pos():
    rng = np.random.default_rng(74)
    T, E, k = 200, 32, 6
    idx = synth.random_routing(rng, T, E, k)
    _, offsets, pos, row_src = oracle.map_routes(idx, E, 8, 24)
    R = int(offsets[-1])
    w = rng.random((T, k)).astype(np.float32)
    rw = oracle.row_weights(pos, w, R + 3)
    ref = np.zeros(R + 3, np.float32)
    for t in range(T):
        for j in range(k):
            if pos[t, j] >= 0:
                ref[pos[t, j]] = w[t, j]
    assert np.array_equal(rw, ref)
    # and through row_src: the weight of row r is that of the slot of token
    # row_src[r] whose position is r
    for r in range(R):
        t = row_src[r]
        j = int(np.nonzero(pos[t] == r)[0][0])
        assert rw[r] == w[t, j]


@pytest.mark.parametrize("weighted", [False, True])
def test_swiglu_quant_transposed_is_the_codec_along_columns(weighted):
    """The transposed output against torch: the fp64 activations' columns in
    blocks of 128 rows, torch fp32 amax/448 of the oracle's fp32 activations
    and torch's float8 cast of the fp32 quotient; and the block-scale bound."""
    rng = np.random.default_rng(75 + weighted)
    R, I = 256, 384
    h = _rows(rng, R, I, scale=3.0)
    rw = rng.uniform(0.05, 2.5, R).astype(np.float32) if weighted else None
    qt, st = oracle.swiglu_quant_t(h, I, rw)
    a = torch.from_numpy(oracle.swiglu_f32(h, I, rw))               # (R, I) fp32
    at = a.t().contiguous().view(I, R // 128, 128)
    amax = at.abs().amax(2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    s_ref = amax / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(st, s_ref.numpy())
    q_ref = (at / s_ref[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(I, R)
    assert np.array_equal(qt, q_ref.numpy())
    a64 = _torch_silu_mul64(h, I, rw).T                              # fp64, (I, R)
    scr = np.repeat(st.astype(np.float64), 128, axis=1)
    deq = oracle.e4m3_to_f64(qt) * scr
    bound = np.maximum(np.abs(a64) * 2.0 ** -4, scr * 2.0 ** -10) * (1 + 2.0 ** -20) \
        + 8 * 2.0 ** -24 * np.abs(a64)
    assert np.all(np.abs(a64 - deq) <= bound)
