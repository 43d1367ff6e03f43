"""GPU parity of tk_swiglu_quant (SwiGLU + 1x128 FP8 quantisation, optionally
weighted by each row's routing weight) against the CPU oracle.

FP8 codes and scales: bit-exact.  Shapes span one block, ragged chunk tails
(I not a multiple of 1024), a device-side row count below the capacity, the
weighted form driven by a real map, codec corners of the activation, and the
DeepSeek-V3 expert shape (65536 rows, I = 2048) compared in full.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def _rows(rng, R, I, gscale=2.0):
    g = synth.normal_f32(rng, (R, I)) * np.float32(gscale)
    u = synth.normal_f32(rng, (R, I))
    return synth.bf16_bits(np.concatenate([g, u], axis=1))


def _map(rng, T, E, k, lo, hi):
    idx = synth.random_routing(rng, T, E, k)
    _, offsets, pos, row_src = oracle.map_routes(idx, E, lo, hi)
    w = rng.uniform(0.01, 1.0, (T, k)).astype(np.float32)
    return pos, row_src, w, int(offsets[-1])


def _check(h, I, got_q, got_s, rows, row_w=None):
    q_ref, s_ref = oracle.swiglu_quant(h[:rows], I, None if row_w is None else row_w[:rows])
    g_q, g_s = got_q[:rows], got_s[:rows]
    bad = np.nonzero((g_q != q_ref).any(1) | (g_s != s_ref).any(1))[0]
    assert bad.size == 0, f"{bad.size} rows differ, first {bad[:5]}"


@pytest.mark.parametrize("R,I", [(64, 128), (100, 384), (257, 1152), (512, 2048), (33, 7168),
                                 # fewer rows than a workgroup's eight: one partial iteration
                                 (1, 128), (3, 2048), (7, 7168),
                                 # 64 scales per row (the most gathered in LDS), 65 and 128
                                 # (stored directly)
                                 (40, 8192), (21, 8320), (9, 16384)])
def test_swiglu_quant_random(R, I):
    rng = np.random.default_rng(R + I)
    h = _rows(rng, R, I)
    q, s = tk.tk_swiglu_quant(to_dev(h, bf16=True))
    torch.cuda.synchronize()
    _check(h, I, to_host(q), to_host(s), R)


@pytest.mark.parametrize("T,E,k,lo,hi,I", [(300, 32, 4, 0, 32, 256), (500, 64, 8, 16, 48, 1152),
                                          (129, 16, 2, 0, 16, 2048), (96, 64, 32, 0, 64, 256),
                                          (150, 32, 12, 8, 30, 384)])
def test_swiglu_quant_weighted_by_map(T, E, k, lo, hi, I):
    rng = np.random.default_rng(T + E + I)
    pos, row_src, w, R = _map(rng, T, E, k, lo, hi)
    cap = R + 5
    h = _rows(rng, cap, I)
    n_rows = torch.tensor([R], dtype=torch.int32, device="cuda")
    rs = np.full(cap, -1, np.int32)
    rs[:R] = row_src
    out = torch.full((cap, I), 0x33, dtype=torch.uint8, device="cuda")
    sc = torch.full((cap, I // 128), -2.0, dtype=torch.float32, device="cuda")
    tk.tk_swiglu_quant(to_dev(h, bf16=True), n_rows, to_dev(rs), to_dev(pos), to_dev(w), out, sc)
    torch.cuda.synchronize()
    g_q, g_s = to_host(out), to_host(sc)
    _check(h, I, g_q, g_s, R, oracle.row_weights(pos, w, R))
    assert np.all(g_q[R:] == 0x33) and np.all(g_s[R:] == -2.0), "wrote rows at or beyond n_rows"


def test_swiglu_quant_corners():
    rng = np.random.default_rng(80)
    I = 1024
    # (activations that overflow fp32 are outside the contract: gates stay
    # small enough that g * u is finite)
    specials = np.array([0.0, -0.0, 20.0, -20.0, 100.0, -100.0, 88.5, -88.5, 1e-30, -3e-5,
                         1.0e30, -65504.0, 0.5, -1.0], np.float32)
    R = 40
    g = rng.choice(specials, (R, I)).astype(np.float32)
    g[::3] = synth.normal_f32(rng, (len(g[::3]), I)) * np.float32(8.0)
    u = synth.normal_f32(rng, (R, I))
    u[1::4] = 0.0
    u[2::4] *= np.float32(1e-20)
    u[3] = rng.choice(specials[:10], I)
    h = synth.bf16_bits(np.concatenate([g, u], axis=1))
    q, s = tk.tk_swiglu_quant(to_dev(h, bf16=True))
    torch.cuda.synchronize()
    _check(h, I, to_host(q), to_host(s), R)


def test_swiglu_quant_zero_rows_and_deterministic():
    rng = np.random.default_rng(81)
    h = to_dev(_rows(rng, 300, 512), bf16=True)
    n0 = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = torch.full((300, 512), 7, dtype=torch.uint8, device="cuda")
    sc = torch.zeros((300, 4), dtype=torch.float32, device="cuda")
    tk.tk_swiglu_quant(h, n0, out=out, scales=sc)
    torch.cuda.synchronize()
    assert np.all(to_host(out) == 7)
    a = [to_host(t) for t in tk.tk_swiglu_quant(h)]
    b = [to_host(t) for t in tk.tk_swiglu_quant(h)]
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


# ------------------------------------------------------------- transposed --
def _check_t(h, I, res, row_w=None):
    out, sc, out_t, sc_t = (to_host(t) for t in res)
    q_ref, s_ref = oracle.swiglu_quant(h, I, row_w)
    qt_ref, st_ref = oracle.swiglu_quant_t(h, I, row_w)
    assert np.array_equal(sc, s_ref) and np.array_equal(out, q_ref), "row-major output"
    assert np.array_equal(sc_t, st_ref), "transposed scales"
    bad = np.argwhere(out_t != qt_ref)
    assert bad.size == 0, f"{len(bad)} transposed codes differ, first {bad[:4]}"


@pytest.mark.parametrize("R,I", [(128, 128), (256, 384), (640, 2048), (128, 7168)])
def test_swiglu_quant_t_random(R, I):
    rng = np.random.default_rng(R * 3 + I)
    h = _rows(rng, R, I)
    res = tk.tk_swiglu_quant_t(to_dev(h, bf16=True))
    torch.cuda.synchronize()
    _check_t(h, I, res)


@pytest.mark.parametrize("T,E,k", [(400, 16, 4), (150, 32, 12), (60, 64, 32)])
def test_swiglu_quant_t_weighted_aligned_map(T, E, k):
    """Rows laid out by the aligned map (segments padded to 128 rows), weights
    through row_src / pos; padding rows have weight 0.  k above 8 takes the
    kernel's extra slot loop."""
    rng = np.random.default_rng(83 + k)
    I = 256
    idx = synth.random_routing(rng, T, E, k)
    _, offsets, pos, row_src = oracle.map_aligned(idx, E, 0, E, 128)
    R = int(offsets[-1])
    assert R % 128 == 0
    w = rng.uniform(0.01, 1.0, (T, k)).astype(np.float32)
    h = _rows(rng, R, I)
    res = tk.tk_swiglu_quant_t(to_dev(h, bf16=True), to_dev(row_src), to_dev(pos), to_dev(w))
    torch.cuda.synchronize()
    _check_t(h, I, res, oracle.row_weights(pos, w, R))


def test_swiglu_quant_t_corners():
    rng = np.random.default_rng(84)
    I, R = 256, 256
    specials = np.array([0.0, -0.0, 20.0, -20.0, 100.0, -100.0, 1e-30, -3e-5, 1.0e30, 0.5],
                        np.float32)
    g = rng.choice(specials, (R, I)).astype(np.float32)
    g[::3] = synth.normal_f32(rng, (len(g[::3]), I)) * np.float32(8.0)
    u = synth.normal_f32(rng, (R, I))
    u[:, 1::4] = 0.0                       # zero columns blocks in the transposed layout
    h = synth.bf16_bits(np.concatenate([g, u], axis=1))
    res = tk.tk_swiglu_quant_t(to_dev(h, bf16=True))
    torch.cuda.synchronize()
    _check_t(h, I, res)


def test_swiglu_quant_t_many_tiles_weighted():
    """More 128x128 tiles (50 x 16 = 800) than the kernel's persistent grid, so
    workgroups take a second tile; weighted through a map of the rows."""
    rng = np.random.default_rng(85)
    R, I = 50 * 128, 2048
    T, k = R // 4, 4
    idx = synth.random_routing(rng, T, 64, k)
    _, offsets, pos, row_src = oracle.map_routes(idx, 64)
    assert int(offsets[-1]) == R
    w = rng.uniform(0.01, 1.0, (T, k)).astype(np.float32)
    h = _rows(rng, R, I)
    res = tk.tk_swiglu_quant_t(to_dev(h, bf16=True), to_dev(row_src), to_dev(pos), to_dev(w))
    torch.cuda.synchronize()
    _check_t(h, I, res, oracle.row_weights(pos, w, R))


# ------------------------------------------------------ sigmoid lookup --
def test_silu_bf16_every_value():
    """RN(g * sigmoid(g)) on all 65536 bf16 values (the SwiGLU kernels' table
    lookup) against the oracle's pinned sigmoid: bit-exact, NaN where NaN."""
    bits = np.arange(0x10000, dtype=np.uint32).astype(np.uint16)
    got = to_host(tk.tk_silu_bf16(to_dev(bits, bf16=True)))
    g = (bits.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore"):
        ref = (g * oracle.sigmoid_f32(g)).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    bad = np.nonzero(got[~nan].view(np.uint32) != ref[~nan].view(np.uint32))[0]
    assert bad.size == 0, f"{bad.size} values differ, first bf16 bits {bits[~nan][bad[:4]]}"
    # and a strided, odd-length call through the grid-stride loop
    many = np.resize(bits, 3 * 65536 + 7)
    got2 = to_host(tk.tk_silu_bf16(to_dev(many, bf16=True)))
    assert np.array_equal(got2.view(np.uint32)[~np.isnan(got2)],
                          np.resize(got, many.size).view(np.uint32)[~np.isnan(got2)])


@pytest.mark.slow
def test_swiglu_v3_expert_shape_full():
    """Both forms at the DeepSeek-V3 expert shape, as launched by the bench:
    65536 expanded rows of the step's routing, I = 2048, weighted by the
    routing weights through the map.  Every code and scale of both layouts is
    compared with the oracle."""
    cfg = synth.v3_gate(0)
    idx, w = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    w = w.astype(np.float32)
    _, offsets, pos, row_src = oracle.map_routes(idx, 256)
    R, I = int(offsets[-1]), 2048
    assert R == 65536
    h = synth.normal_bf16(np.random.default_rng(86), (R, 2 * I))
    h_d, rs_d, pos_d, w_d = to_dev(h, bf16=True), to_dev(row_src), to_dev(pos), to_dev(w)
    q, s = tk.tk_swiglu_quant(h_d, None, rs_d, pos_d, w_d)
    res_t = tk.tk_swiglu_quant_t(h_d, rs_d, pos_d, w_d)
    torch.cuda.synchronize()
    del h_d
    rw = oracle.row_weights(pos, w, R)
    q_ref, s_ref = oracle.swiglu_quant(h, I, rw)
    g_q = to_host(q)
    bad = np.nonzero((g_q != q_ref).any(1))[0]
    assert bad.size == 0, f"plain form: {bad.size} rows of codes differ, first {bad[:4]}"
    assert np.array_equal(to_host(s), s_ref), "plain form: scales"
    out, sc, out_t, sc_t = (to_host(t) for t in res_t)
    assert np.array_equal(out, q_ref) and np.array_equal(sc, s_ref), "transposing form: row-major"
    del q_ref, g_q, out
    qt_ref, st_ref = oracle.swiglu_quant_t(h, I, rw)
    assert np.array_equal(sc_t, st_ref), "transposing form: transposed scales"
    bad = np.nonzero((out_t != qt_ref).any(1))[0]
    assert bad.size == 0, f"transposing form: {bad.size} columns of codes differ, first {bad[:4]}"


@pytest.mark.parametrize("seed", range(32))
def test_swiglu_sweep(seed):
    """Seeded random shapes for both forms: I any multiple of 128 up to 2048,
    weighted through a random map or not; the plain form with a device-side
    row count below its capacity, the transposing form over the map's rows
    rounded up to whole 128-row blocks (extra rows unweighted: weight 0)."""
    rng = np.random.default_rng(8000 + seed)
    I = 128 * int(rng.integers(1, 17))
    T = int(rng.integers(1, 400))
    E = int(rng.choice([8, 16, 64]))
    k = int(rng.integers(1, min(E, 8) + 1))
    lo = int(rng.integers(0, E))
    hi = int(rng.integers(lo + 1, E + 1))
    pos, row_src, w, R = _map(rng, T, E, k, lo, hi)
    weighted = bool(rng.integers(0, 2))
    # plain form
    cap = R + int(rng.integers(0, 40)) + 1
    h = _rows(rng, cap, I, gscale=float(rng.choice([1.0, 3.0, 8.0])))
    rs = np.full(cap, -1, np.int32)
    rs[:R] = row_src
    n_rows = torch.tensor([R], dtype=torch.int32, device="cuda")
    args = (to_dev(rs), to_dev(pos), to_dev(w)) if weighted else (None, None, None)
    q, s = tk.tk_swiglu_quant(to_dev(h, bf16=True), n_rows, *args)
    torch.cuda.synchronize()
    rw = oracle.row_weights(pos, w, cap) if weighted else None
    _check(h, I, to_host(q), to_host(s), R, rw)
    # transposing form
    Rt = max(128, (R + 127) // 128 * 128)
    ht = _rows(rng, Rt, I)
    rst = np.full(Rt, -1, np.int32)
    rst[:R] = row_src
    args = (to_dev(rst), to_dev(pos), to_dev(w)) if weighted else (None, None, None)
    res = tk.tk_swiglu_quant_t(to_dev(ht, bf16=True), *args)
    torch.cuda.synchronize()
    _check_t(ht, I, res, oracle.row_weights(pos, w, Rt) if weighted else None)
