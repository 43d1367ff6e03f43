"""GPU parity of tk_quant (power-of-two 1x128 FP8, 128x128 FP8, per-channel
FP8, FP4 E2M1 1x32) against the CPU oracle: codes and scales bit-exact.

Shapes cover ragged tails (columns not a multiple of a wave's chunk, rows not
a multiple of a tile or chunk), codec corners (every bf16 magnitude up to 448,
E2M1 midpoints and their neighbours after scaling, zeros, signed zeros,
clamped blocks, outliers) and the DeepSeek-V3 hidden-state shape.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")

MODES = [tk.TK_QUANT_FP8_1X128, tk.TK_QUANT_FP8_1X128_POW2, tk.TK_QUANT_FP8_128X128,
         tk.TK_QUANT_FP8_PER_CHANNEL, tk.TK_QUANT_FP4_1X32]


def _matrix(rng, rows, cols):
    x = synth.normal_f32(rng, (rows, cols))
    x[::5] *= np.float32(40.0)
    x[1::7] *= np.float32(1e-6)
    x[2 % rows, : min(cols, 64)] = 0.0
    x[3 % rows, 5::9] = -0.0
    return synth.bf16_bits(x)


def _check(x, mode):
    q, s = tk.tk_quant(to_dev(x, bf16=True), mode)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant(x, mode)
    g_q, g_s = to_host(q), to_host(s)
    assert np.array_equal(g_s, s_ref), f"scales differ at {np.argwhere(g_s != s_ref)[:4]}"
    bad = np.argwhere(g_q != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:4]}"


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 384), (130, 1152), (300, 2048), (5, 7168),
                                       (2, 65536), (129, 16384), (3000, 128)])
def test_quant_random(mode, rows, cols):
    _check(_matrix(np.random.default_rng(rows * 31 + cols + mode), rows, cols), mode)


@pytest.mark.parametrize("mode", MODES)
def test_quant_codec_corners(mode):
    # every positive bf16 magnitude <= 448, both signs, 127 per 128-block
    # after a block maximum of 448, so scale 1 (FP8) lands on exact codes
    allb = np.arange(0, 0x8000, dtype=np.uint32)
    vals = (allb << 16).view(np.float32)
    vals = vals[np.isfinite(vals) & (np.abs(vals) <= 448.0)]
    vals = np.concatenate([vals, -vals])
    n_blocks = int(np.ceil(vals.size / 127))
    blocks = np.zeros((n_blocks, 128), np.float32)
    blocks[:, 0] = 448.0
    flat = blocks[:, 1:].reshape(-1)
    flat[: vals.size] = vals
    blocks[:, 1:] = flat.reshape(n_blocks, 127)
    cols = 1024
    rows = int(np.ceil(n_blocks * 128 / cols))
    m = np.zeros(rows * cols, np.float32)
    m[: n_blocks * 128] = blocks.reshape(-1)
    _check(synth.bf16_bits(m.reshape(rows, cols)), mode)


def test_fp4_midpoints():
    # block maximum 4 -> scale 1: values at the E2M1 midpoints, their bf16
    # neighbours, and saturating magnitudes, in every position of the block
    mids = np.float32([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 6.0, 7.5])
    up = (mids.view(np.uint32) + 0x10000).view(np.float32)
    dn = (mids.view(np.uint32) - 0x10000).view(np.float32)
    v = np.concatenate([mids, up, dn, -mids, -up, -dn])
    rows = 64
    x = np.resize(v, (rows, 256)).astype(np.float32)
    x[:, ::32] = 7.9                      # block maximum in [4, 8): scale 2^0
    x = synth.bf16_bits(x)
    _check(x, tk.TK_QUANT_FP4_1X32)
    q, s = oracle.quant(x, tk.TK_QUANT_FP4_1X32)
    assert np.all(s == 1.0)


@pytest.mark.parametrize("mode", MODES)
def test_quant_v3_hidden_full(mode):
    _check(synth.v3_hidden(0), mode)


def test_quant_128x128_weight_shape():
    # a (4096 x 7168) weight-shaped matrix with a ragged last tile row
    x = synth.normal_bf16(np.random.default_rng(65), (4096 + 40, 7168))
    _check(x, tk.TK_QUANT_FP8_128X128)


def test_quant_zero_rows_and_deterministic():
    x = to_dev(_matrix(np.random.default_rng(66), 200, 512), bf16=True)
    for mode in MODES:
        a = [to_host(t) for t in tk.tk_quant(x, mode)]
        b = [to_host(t) for t in tk.tk_quant(x, mode)]
        assert all(np.array_equal(u, v) for u, v in zip(a, b)), mode
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    tk.tk_quant(e, tk.TK_QUANT_FP8_PER_CHANNEL)
    torch.cuda.synchronize()


_ALIGN = {tk.TK_QUANT_FP8_1X128: 128, tk.TK_QUANT_FP8_1X128_POW2: 128,
          tk.TK_QUANT_FP8_128X128: 128, tk.TK_QUANT_FP8_PER_CHANNEL: 8, tk.TK_QUANT_FP4_1X32: 32}


@pytest.mark.parametrize("seed", range(32))
def test_quant_sweep(seed):
    """Seeded random shapes: any mode, 1..600 rows, columns any allowed multiple up to 4096."""
    rng = np.random.default_rng(7000 + seed)
    mode = MODES[int(rng.integers(len(MODES)))]
    a = _ALIGN[mode]
    rows = int(rng.integers(1, 601))
    cols = a * int(rng.integers(1, 4096 // a + 1))
    _check(_matrix(rng, rows, cols), mode)
