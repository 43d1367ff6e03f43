"""Pins of the oracle's other codec granularities: power-of-two 1x128 FP8
scales, 128x128 per-block FP8, per-channel FP8 and 1x32 FP4 (E2M1) with
power-of-two scales.

FP8 codes against torch's float8_e4m3fn cast of torch's fp32 quotient, scales
against torch fp32 amax/448 (tile / column reductions by reshape and amax);
power-of-two scales against their defining inequalities in fp64; E2M1 against
a brute-force nearest-value search with ties to the even code, written here in
numpy, and the block exponent against numpy's frexp.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth

Q = oracle


def _f32(bits16):
    return (np.asarray(bits16, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _matrix(rng, rows, cols):
    x = synth.normal_f32(rng, (rows, cols))
    x[::5] *= np.float32(40.0)
    x[1::7] *= np.float32(1e-6)                      # tiny (clamped) blocks
    x[2, :64] = 0.0
    return synth.bf16_bits(x)


def _cast(v32):
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def test_pow2_scale_is_the_smallest_power_of_two():
    bits = np.arange(0x0001, 0x7F80, 7, dtype=np.uint32)           # positive bf16 magnitudes
    amax = (bits << 16).view(np.float32)
    for a in np.concatenate([amax, np.float32([448.0, 449.0, 392.0, 896.0, 1e-4, 0.0])]):
        s = Q.pow2_scale_e4m3(a)
        m, e = np.frexp(s)
        assert m == 0.5                                             # a power of two
        ac = max(float(a), float(np.float32(1e-4)))
        assert 448.0 * s >= ac and 448.0 * s / 2 < ac, (a, s)


@pytest.mark.parametrize("pow2", [0, 1])
def test_quant_1x128_matches_torch(pow2):
    rng = np.random.default_rng(60 + pow2)
    x = _matrix(rng, 50, 1024)
    q, sc = Q.quant(x, Q.QUANT_FP8_1X128_POW2 if pow2 else Q.QUANT_FP8_1X128)
    xf = torch.from_numpy(_f32(x)).view(50, 8, 128)
    amax = xf.abs().amax(2).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    if pow2:
        e = torch.ceil(torch.log2(amax.double() / 448.0))
        s_ref = torch.pow(2.0, e)
        s_ref = torch.where(448.0 * s_ref / 2 >= amax.double(), s_ref / 2, s_ref)   # log2 rounding
        s_ref = torch.where(448.0 * s_ref < amax.double(), s_ref * 2, s_ref).float()
    else:
        s_ref = amax / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(sc, s_ref.numpy())
    q_ref = _cast((xf / s_ref[:, :, None]).reshape(50, 1024).numpy())
    assert np.array_equal(q, q_ref)
    if not pow2:
        assert np.array_equal((q, sc)[0], oracle.quant_row(x)[0])


@pytest.mark.parametrize("rows", [128, 300, 5])
def test_quant_128x128_matches_torch(rows):
    rng = np.random.default_rng(rows)
    cols = 512
    x = _matrix(rng, rows, cols)
    q, sc = Q.quant(x, Q.QUANT_FP8_128X128)
    tr = (rows + 127) // 128
    pad = np.zeros((tr * 128, cols), np.float32)
    pad[:rows] = _f32(x)
    t = torch.from_numpy(pad).view(tr, 128, cols // 128, 128)
    amax = t.abs().amax(dim=(1, 3)).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    s_ref = amax / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(sc, s_ref.numpy())
    div = (t / s_ref[:, None, :, None]).reshape(tr * 128, cols)[:rows]
    assert np.array_equal(q, _cast(div.numpy()))


def test_quant_per_channel_matches_torch():
    rng = np.random.default_rng(62)
    x = _matrix(rng, 333, 256)
    x[:, 7] = 0                                              # an all-zero column: clamped
    q, sc = Q.quant(x, Q.QUANT_FP8_PER_CHANNEL)
    xf = torch.from_numpy(_f32(x))
    amax = xf.abs().amax(0).clamp_min(torch.tensor(1e-4, dtype=torch.float32))
    s_ref = amax / torch.tensor(448.0, dtype=torch.float32)
    assert np.array_equal(sc, s_ref.numpy())
    assert np.array_equal(q, _cast((xf / s_ref[None, :]).numpy()))


# ------------------------------------------------------------------- FP4 --
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _e2m1_brute(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - E2M1[None, :])
    best = np.zeros(v.shape, np.int64)
    for c in range(1, 8):
        better = (d[:, c] < d[np.arange(v.size), best]) | \
                 ((d[:, c] == d[np.arange(v.size), best]) & (c % 2 == 0))
        best = np.where(better, c, best)
    best = np.where(a >= 6.0, 7, best)
    return (best | np.where(np.signbit(v), 8, 0)).astype(np.uint8)


def test_e2m1_encoder_brute_force():
    rng = np.random.default_rng(63)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    near = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 10)])
    v = np.concatenate([near, -near, E2M1.astype(np.float32), -E2M1.astype(np.float32),
                        rng.uniform(-8, 8, 100000).astype(np.float32),
                        np.float32([0.0, -0.0, 6.0, 7.0, 1e9, -1e9, 1e-30])])
    assert np.array_equal(Q.e2m1_from_f32(v), _e2m1_brute(v))
    # ties go to the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 2.5 -> 2, 5 -> 4
    assert list(Q.e2m1_from_f32(mids)) == [0, 2, 2, 4, 4, 6, 6]
    assert Q.e2m1_from_f32(np.float32([-0.0]))[0] == 8
    assert np.array_equal(Q.e2m1_to_f64(np.arange(8)), E2M1)


def test_quant_fp4_1x32_reference_and_bounds():
    rng = np.random.default_rng(64)
    rows, cols = 40, 256
    x = _matrix(rng, rows, cols)
    q, sc = Q.quant(x, Q.QUANT_FP4_1X32)
    xf = _f32(x).reshape(rows, cols // 32, 32)
    amax = np.maximum(np.abs(xf).max(2), np.float32(1e-4))
    _, e = np.frexp(amax)
    s_ref = np.ldexp(np.float32(1.0), e - 1 - 2).astype(np.float32)
    assert np.array_equal(sc, s_ref)
    v = (xf / s_ref[:, :, None]).astype(np.float32).reshape(-1)
    codes = _e2m1_brute(v).reshape(rows, cols)
    assert np.array_equal(q, (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    # amax / X in [4, 8): the block's largest magnitude lands on 4 or 6
    r = amax / s_ref
    assert np.all((r >= 4) & (r < 8))
    deq = Q.e2m1_to_f64(codes).reshape(rows, cols // 32, 32) * s_ref[:, :, None]
    err = np.abs(xf.astype(np.float64) - deq)
    assert np.all(err <= 2.0 * s_ref[:, :, None])            # worst: 8X-eps saturated to 6X
