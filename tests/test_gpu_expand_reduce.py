"""GPU parity of tk_expand_quant, tk_expert_standin and tk_reduce against the
CPU oracle.

FP8 codes and scales, bf16 copies and stand-in outputs: bit-exact.  Combine:
|gpu - ref| <= 1e-2 + 1e-2*|ref| per element (the fraction of bit-identical
elements is reported and expected to be high).
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import combine_report, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def _routing(T, E, k, seed, lo=0, hi=None):
    rng = np.random.default_rng(seed)
    idx = synth.random_routing(rng, T, E, k)
    counts, offsets, pos, row_src = oracle.map_routes(idx, E, lo, E if hi is None else hi)
    return idx, pos, int(offsets[-1])


def _special_rows(H):
    """Rows that hit the codec's corners: zeros, signed zeros, clamped tiny
    blocks, blocks with scale exactly 1 holding every bf16 magnitude <= 448,
    E4M3 midpoints (ties) and their bf16 neighbours, huge values."""
    rows = [np.zeros(H, np.float32), np.full(H, -0.0, np.float32)]
    t = np.full(H, 3e-5, np.float32); t[1::2] *= -1; rows.append(t)
    # every bf16 pattern with magnitude <= 448, packed 127 per block + one 448
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
    per_row = H // 128
    n_rows = int(np.ceil(n_blocks / per_row))
    pad = np.zeros((n_rows * per_row - n_blocks, 128), np.float32)
    pad[:, 0] = 448.0
    rows.extend(np.concatenate([blocks, pad]).reshape(n_rows, H))
    # scales that are not powers of two: amax 300, 1.7, 1e-3 with ramps
    for amax in (300.0, 1.7, 1e-3, 6.0e4):
        r = np.linspace(-amax, amax, H).astype(np.float32)
        rows.append(r)
    return synth.bf16_bits(np.stack(rows))


def _describe(x_bits, g_row, o_row, scale):
    d = np.nonzero(g_row != o_row)[0][:4]
    xs = oracle.bf16_to_f32(x_bits[d])
    return [(int(c), float(xs[i]), float(scale[c // 128]), hex(g_row[c]), hex(o_row[c]))
            for i, c in enumerate(d)]


def _check_expand_fp8(x_bits, pos, R):
    T, H = x_bits.shape
    xq, sc = tk.tk_expand_quant(to_dev(x_bits, bf16=True), to_dev(pos), tk.TK_EXPAND_FP8_E4M3_1X128, R)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_row(x_bits)           # per token, once
    g_q, g_s = to_host(xq), to_host(sc)
    for j in range(pos.shape[1]):
        valid = pos[:, j] >= 0
        rows = pos[valid, j]
        bad = np.nonzero((g_q[rows] != q_ref[valid]).any(1))[0]
        if bad.size:
            t = int(np.nonzero(valid)[0][bad[0]])
            detail = _describe(x_bits[t], g_q[pos[t, j]], q_ref[t], s_ref[t])
            raise AssertionError(f"slot {j}: FP8 bytes differ for {bad.size} tokens, first t={t}: "
                                 f"(col, x, scale, gpu, oracle) {detail}")
        assert np.array_equal(g_s[rows], s_ref[valid]), f"slot {j}: scales differ"


@pytest.mark.parametrize("T,E,k,H", [(64, 16, 2, 256), (100, 32, 3, 1152), (513, 64, 8, 7168),
                                     (37, 8, 1, 128), (200, 16, 4, 3072), (60, 64, 32, 1024)])
def test_expand_fp8_random(T, E, k, H):
    idx, pos, R = _routing(T, E, k, T + H)
    rng = np.random.default_rng(H)
    x = synth.normal_bf16(rng, (T, H))
    x[::7] = synth.bf16_bits(synth.normal_f32(rng, (len(x[::7]), H)) * np.float32(50.0))
    _check_expand_fp8(x, pos, R)


@pytest.mark.parametrize("H", [1024, 7168])
def test_expand_fp8_codec_corners(H):
    x = _special_rows(H)
    T = x.shape[0]
    pos = np.arange(T, dtype=np.int32)[:, None]
    _check_expand_fp8(x, pos, T)


def test_expand_fp8_quotient_just_above_448():
    """Every bf16 block maximum m >= 1e-4 whose quotient m / RN(m/448) rounds
    above 448 in fp32 (about 9 % of them): the code must still be 448."""
    h = np.arange(0x3800, 0x7F80, dtype=np.uint32)
    a = (h << 16).view(np.float32)
    a = a[a >= np.float32(1e-4)]
    over = a[(a / (a / np.float32(448.0)).astype(np.float32)).astype(np.float32) > 448.0]
    assert over.size > 1000
    H = 1024
    rng = np.random.default_rng(50)
    blocks = rng.uniform(-1, 1, (over.size, 128)).astype(np.float32) * over[:, None]
    blocks[:, 0] = over
    blocks[1::2, 0] *= -1                                  # negative maxima too
    n_rows = int(np.ceil(over.size / (H // 128)))
    pad = np.ones((n_rows * (H // 128) - over.size, 128), np.float32)
    x = synth.bf16_bits(np.concatenate([blocks, pad]).reshape(n_rows, H))
    pos = np.arange(n_rows, dtype=np.int32)[:, None]
    _check_expand_fp8(x, pos, n_rows)


def test_expand_fp8_v3_full():
    cfg = synth.v3_gate(0)
    idx, _ = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    _, offsets, pos, _ = oracle.map_routes(idx, 256)
    x = synth.v3_hidden(0)
    _check_expand_fp8(x, pos, int(offsets[-1]))


def test_expand_skips_and_capacity():
    T, E, k, H = 300, 16, 4, 512
    idx, pos, R = _routing(T, E, k, 11, lo=4, hi=12)     # masked routes have pos -1
    cap = R - 5                                            # last rows beyond capacity
    x = synth.normal_bf16(np.random.default_rng(12), (T, H))
    sentinel = 0x5A
    out = torch.full((cap + 3, H), sentinel, dtype=torch.uint8, device="cuda")
    sc = torch.full((cap + 3, H // 128), -1.0, dtype=torch.float32, device="cuda")
    tk.tk_expand_quant(to_dev(x, bf16=True), to_dev(pos), tk.TK_EXPAND_FP8_E4M3_1X128, cap,
                       out=out, scales=sc)
    ref_q, ref_s = oracle.expand(x, pos, 1, cap)
    g = to_host(out)
    assert np.array_equal(g[:cap], ref_q) and np.array_equal(to_host(sc)[:cap], ref_s)
    assert np.all(g[cap:] == sentinel), "wrote beyond rows_capacity"


@pytest.mark.parametrize("T,E,k,H", [(64, 16, 2, 256), (129, 8, 3, 520), (10, 4, 1, 8),
                                     (300, 64, 8, 7168), (50, 64, 32, 512)])
def test_expand_bf16(T, E, k, H):
    idx, pos, R = _routing(T, E, k, T * 3 + H)
    x = synth.normal_bf16(np.random.default_rng(T), (T, H))
    out, _ = tk.tk_expand_quant(to_dev(x, bf16=True), to_dev(pos), tk.TK_EXPAND_BF16, R)
    ref, _ = oracle.expand(x, pos, 0, R)
    assert np.array_equal(to_host(out), ref)


def test_expand_bf16_v3_full():
    # the expand without quantisation at the bench's shape: every one of the
    # 65536 rows a bitwise copy of its token
    cfg = synth.v3_gate(0)
    idx, _ = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    _, offsets, pos, _ = oracle.map_routes(idx, 256)
    x = synth.v3_hidden(0)
    R = int(offsets[-1])
    out, _ = tk.tk_expand_quant(to_dev(x, bf16=True), to_dev(pos), tk.TK_EXPAND_BF16, R)
    torch.cuda.synchronize()
    ref, _ = oracle.expand(x, pos, 0, R)
    assert np.array_equal(to_host(out), ref)


def test_expand_zero_tokens():
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    pos = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    tk.tk_expand_quant(x, pos, tk.TK_EXPAND_FP8_E4M3_1X128, 0)
    torch.cuda.synchronize()


def test_standin_matches_oracle():
    T, E, k, H = 400, 16, 3, 1024
    idx, pos, R = _routing(T, E, k, 21)
    x = synth.normal_bf16(np.random.default_rng(22), (T, H))
    xq, sc = tk.tk_expand_quant(to_dev(x, bf16=True), to_dev(pos), tk.TK_EXPAND_FP8_E4M3_1X128, R + 7)
    n_rows = torch.tensor([R], dtype=torch.int32, device="cuda")
    y = tk.tk_expert_standin(xq, sc, n_rows, 0.5)
    torch.cuda.synchronize()
    q, s = oracle.expand(x, pos, 1, R)
    ref = oracle.standin(q, s, 0.5)
    assert np.array_equal(to_host(y)[:R], ref)


# ------------------------------------------------------------------ reduce --
def _check_reduce(y_bits, pos, w, sample=None, fn="tk_reduce"):
    out = getattr(tk, fn)(to_dev(y_bits, bf16=True), to_dev(pos), to_dev(w))
    torch.cuda.synchronize()
    g = to_host(out)
    if sample is None:
        ref = oracle.reduce(y_bits, pos, w)
    else:
        ref = oracle.reduce(y_bits, pos[sample], w[sample])
        g = g[sample]
    rep = combine_report(g, ref)
    assert rep["ok"], rep
    assert rep["bit_exact_frac"] > 0.98, rep
    return rep


@pytest.mark.parametrize("T,E,k,H", [(64, 16, 2, 256), (333, 32, 8, 1032), (50, 8, 1, 128),
                                     (77, 64, 6, 7168), (40, 64, 12, 512), (45, 64, 32, 1032)])
def test_reduce_random(T, E, k, H):
    idx, pos, R = _routing(T, E, k, T + k)
    rng = np.random.default_rng(H + k)
    y = synth.normal_bf16(rng, (R, H))
    w = rng.random((T, k)).astype(np.float32)
    _check_reduce(y, pos, w)


@pytest.mark.parametrize("T", [1, 2, 3, 5])
@pytest.mark.parametrize("k", [1, 4, 8])
def test_reduce_few_tokens(T, k):
    # a handful of tokens: fewer waves than the grid's first workgroup row,
    # odd counts, k of one slot and of the compiled sizes
    H = 1032
    rng = np.random.default_rng(100 * T + k)
    R = T * k
    pos = rng.permutation(R).astype(np.int32).reshape(T, k)
    pos[rng.random((T, k)) < 0.25] = -1      # some masked slots
    y = synth.normal_bf16(rng, (R, H))
    w = rng.random((T, k)).astype(np.float32)
    _check_reduce(y, pos, w)


# tk_reduce_dense: for rows of at least four 512-column units and T >=
# (compute units) x 16 it takes its staged form (a workgroup combines up to 16
# consecutive tokens, keeps the results in registers and stores its rows as
# one burst after a barrier), in rounds of one workgroup per CU with the
# tokens spread evenly over them (on 256 CUs: T=4500 -> 9 tokens per
# workgroup, 256 + 244 workgroups; T=5333 -> 11, 256 + 229), one launch per
# round when a round moves at least 480 MiB (k=8, H=7168: T=8191 -> 16
# tokens, launches of 256 + 256 workgroups, the last one short a token;
# T=9000 -> 12 tokens, 256 + 256 + 238); shorter rows, tk_reduce, slices of
# 1000 tokens and T just below the threshold take the one-wave-per-unit
# kernel.  Per token the arithmetic is the same, so all must agree bit for
# bit; both stay within the combine tolerance of the oracle.  Cases: every
# compiled k, ragged last workgroups, rounds and launches, a 520-column row
# (a partly filled 512-column unit), masked slots and rows beyond y.
@pytest.mark.parametrize("T,k,H", [(4096, 8, 7168), (4100, 8, 1024), (5000, 6, 2048),
                                   (4500, 4, 4096), (4600, 2, 520), (4097, 1, 2048),
                                   (4111, 6, 7168), (5333, 4, 7168), (4095, 8, 7168),
                                   (4500, 8, 4096), (10000, 8, 1024), (12289, 4, 3072),
                                   (8191, 8, 7168), (9000, 8, 7168), (4400, 2, 2056),
                                   # runtime k: the one-wave-per-unit kernel for both
                                   (4096, 12, 1024), (4200, 32, 520)])
def test_reduce_dense_equals_reduce(T, k, H):
    rng = np.random.default_rng(T + 10 * k + H)
    R = T * k
    pos = rng.permutation(R).astype(np.int32).reshape(T, k)
    pos[rng.random((T, k)) < 0.1] = -1                      # masked slots
    rows = R - R // 50                                      # the last rows are beyond y
    y = synth.normal_bf16(rng, (rows, H))
    w = rng.random((T, k)).astype(np.float32)
    yd, pd, wd = to_dev(y, bf16=True), to_dev(pos), to_dev(w)
    dense = to_host(tk.tk_reduce_dense(yd, pd, wd))
    plain = to_host(tk.tk_reduce(yd, pd, wd))
    sliced = np.concatenate([to_host(tk.tk_reduce_dense(yd, pd[a:a + 1000], wd[a:a + 1000]))
                             for a in range(0, T, 1000)])
    assert np.array_equal(dense, plain)
    assert np.array_equal(dense, sliced)
    sample = np.random.default_rng(T).choice(T, 300, replace=False)
    ref = oracle.reduce(y, pos[sample], w[sample])
    rep = combine_report(dense[sample], ref)
    assert rep["ok"] and rep["bit_exact_frac"] > 0.98, rep


def test_reduce_dense_with_rows_cut_short():
    # a short y (rows < T*k): the slots pointing past its end are skipped by
    # both forms, as if masked -- a fifth of the rows are missing here
    T, k, H = 4096, 8, 2048
    rng = np.random.default_rng(77)
    pos = rng.permutation(T * k).astype(np.int32).reshape(T, k)
    rows = T * k * 4 // 5
    y = synth.normal_bf16(rng, (rows, H))
    w = rng.random((T, k)).astype(np.float32)
    yd, pd, wd = to_dev(y, bf16=True), to_dev(pos), to_dev(w)
    dense = to_host(tk.tk_reduce_dense(yd, pd, wd))
    assert np.array_equal(dense, to_host(tk.tk_reduce(yd, pd, wd)))
    sample = np.random.default_rng(78).choice(T, 200, replace=False)
    rep = combine_report(dense[sample], oracle.reduce(y, pos[sample], w[sample]))
    assert rep["ok"] and rep["bit_exact_frac"] > 0.98, rep


def test_reduce_masked_and_empty_tokens():
    T, E, k, H = 400, 64, 8, 1024
    idx, pos, R = _routing(T, E, k, 31, lo=32, hi=40)
    rng = np.random.default_rng(32)
    y = synth.normal_bf16(rng, (max(R, 1), H))
    w = rng.random((T, k)).astype(np.float32)
    assert (pos < 0).all(1).any(), "want tokens without local routes"
    rep = _check_reduce(y, pos, w)
    out = to_host(tk.tk_reduce(to_dev(y, bf16=True), to_dev(pos), to_dev(w)))
    assert np.all(out[(pos < 0).all(1)] == 0)


def test_reduce_exact_gather():
    T, H = 256, 2048
    y = synth.normal_bf16(np.random.default_rng(33), (T, H))
    perm = np.random.default_rng(34).permutation(T).astype(np.int32)[:, None]
    out = tk.tk_reduce(to_dev(y, bf16=True), to_dev(perm), to_dev(np.ones((T, 1), np.float32)))
    assert np.array_equal(to_host(out), y[perm[:, 0]])


@pytest.mark.slow
@pytest.mark.parametrize("fn", ["tk_reduce", "tk_reduce_dense"])   # the bench's step takes the second
def test_reduce_v3_full(fn):
    # the weighted combine at the DeepSeek-V3 shape: expert outputs (65536,
    # 7168) through the oracle's routing of the v3 gating workload, every one
    # of the 8192 output tokens compared with the oracle
    cfg = synth.v3_gate(0)
    idx, w = oracle.route(cfg["logits"], cfg["bias"], cfg["k"], **cfg["route"])
    _, offsets, pos, _ = oracle.map_routes(idx, 256)
    y = synth.v3_expert_out(0)
    rep = _check_reduce(y, pos, w.astype(np.float32), None, fn)
    print(f"{fn} v3 full: {rep}")
