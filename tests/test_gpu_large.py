"""GPU parity past 4 GiB: the routing step, the SwiGLU and the codecs at T = 76800 tokens,
H = 7168, E = 256, k = 8 (R = 614,400 expanded rows).  The FP8 expand writes
4.4 GB, the bf16 expand and the combine's input y are 8.8 GB and the SwiGLU
reads 5.0 GB, so their byte offsets pass 2^32 and need 64-bit arithmetic.

Route and map are compared with the oracle in full.  The expand, the combine
and the SwiGLU are compared on sampled tokens, rows and 128-row blocks,
always including the ones at the highest addresses (the last rows of the
expert-contiguous layout, the last token, the last row block).  The large
inputs (x, y) are drawn on the GPU by torch's seeded generator and the sampled
parts copied back for the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import W_ATOL, W_RTOL, combine_report, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")

T, H, E, K = 76800, 7168, 256, 8
R = T * K
I = 2048


def _gpu_bf16(shape, seed, dev):
    """N(0, 1) bf16 drawn on the device in 2^27-element pieces (no fp32 copy
    of the whole tensor)."""
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
    flat = out.view(-1)
    step = 1 << 27
    for s in range(0, flat.numel(), step):
        n = min(step, flat.numel() - s)
        flat[s:s + n] = torch.randn(n, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    return out


def _bits(t):
    """bf16 device tensor -> uint16 host array."""
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.fixture(scope="module")
def big():
    dev = torch.device("cuda:0")
    gate = synth.v3_gate(1, T=T)
    logits, bias, r = gate["logits"], gate["bias"], gate["route"]
    o_idx, o_w = oracle.route(logits, bias, K, **r)
    oc, oo, opos, ors = oracle.map_routes(o_idx, E)
    assert int(oo[-1]) == R
    rng = np.random.default_rng(7)
    # tokens whose rows are the last rows, the last token, and random ones
    last_rows = np.unique(ors[R - 12:])
    sample = np.unique(np.concatenate([last_rows, [0, T - 1], rng.choice(T, 48, replace=False)]))
    d = dict(dev=dev, logits=logits, bias=bias, route=r, o_idx=o_idx, o_w=o_w, oc=oc, oo=oo,
             opos=opos, ors=ors, sample=sample, rng=rng)
    yield d
    d.clear()
    torch.cuda.empty_cache()


def test_large_route_and_map(big):
    idx, w = tk.tk_route(to_dev(big["logits"]), to_dev(big["bias"]), K, tk.RouteOpts(**big["route"]))
    torch.cuda.synchronize()
    g_idx, g_w = to_host(idx), to_host(w)
    bad = np.nonzero((g_idx != big["o_idx"]).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens differ, first {bad[:5]}"
    assert np.allclose(g_w, big["o_w"], rtol=W_RTOL, atol=W_ATOL)
    counts, offsets, pos, row_src = tk.tk_map(to_dev(big["o_idx"]), E)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(counts), big["oc"])
    assert np.array_equal(to_host(offsets), big["oo"])
    assert np.array_equal(to_host(pos), big["opos"])
    assert np.array_equal(to_host(row_src), big["ors"])


def test_large_expand_fp8_and_bf16(big):
    dev, sample, opos = big["dev"], big["sample"], big["opos"]
    x = _gpu_bf16((T, H), 11, dev)
    pos = to_dev(opos)
    xq = torch.empty((R, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((R, H // 128), dtype=torch.float32, device=dev)
    tk.tk_expand_quant(x, pos, tk.TK_EXPAND_FP8_E4M3_1X128, R, xq, sc)
    torch.cuda.synchronize()
    x_s = _bits(x[torch.from_numpy(sample).to(dev)])
    q_ref, s_ref = oracle.quant_row(x_s)
    rows = torch.from_numpy(opos[sample].reshape(-1).astype(np.int64)).to(dev)
    g_q = to_host(xq[rows]).reshape(len(sample), K, H)
    g_s = to_host(sc[rows]).reshape(len(sample), K, H // 128)
    for j in range(K):
        assert np.array_equal(g_q[:, j], q_ref), f"FP8 codes, slot {j}"
        assert np.array_equal(g_s[:, j], s_ref), f"scales, slot {j}"
    del xq, sc
    xe = torch.empty((R, H), dtype=torch.bfloat16, device=dev)
    tk.tk_expand_quant(x, pos, tk.TK_EXPAND_BF16, R, xe)
    torch.cuda.synchronize()
    g_e = _bits(xe[rows]).reshape(len(sample), K, H)
    for j in range(K):
        assert np.array_equal(g_e[:, j], x_s), f"bf16 rows, slot {j}"
    del xe, x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fn", ["tk_reduce_dense", "tk_reduce"])
def test_large_combine(big, fn):
    dev, sample, opos = big["dev"], big["sample"], big["opos"]
    y = _gpu_bf16((R, H), 12, dev)
    w = big["rng"].uniform(0.05, 0.6, (T, K)).astype(np.float32)
    out = getattr(tk, fn)(y, to_dev(opos), to_dev(w))
    torch.cuda.synchronize()
    if fn == "tk_reduce_dense":
        # every token against the one-wave-per-unit kernel (the same arithmetic;
        # here the dense form runs 19 launches of 256 workgroups)
        assert torch.equal(out, tk.tk_reduce(y, to_dev(opos), to_dev(w))), "dense != plain"
    # the sampled tokens' rows, renumbered 0.. for the oracle
    rows = opos[sample].reshape(-1)
    y_s = _bits(y[torch.from_numpy(rows.astype(np.int64)).to(dev)])
    pos_s = np.arange(rows.size, dtype=np.int32).reshape(len(sample), K)
    ref = oracle.reduce(y_s, pos_s, w[sample])
    rep = combine_report(_bits(out[torch.from_numpy(sample).to(dev)]), ref)
    assert rep["ok"], rep
    del y, out
    torch.cuda.empty_cache()


def test_large_swiglu_both_layouts(big):
    dev, opos = big["dev"], big["opos"]
    h = _gpu_bf16((R, 2 * I), 13, dev)
    w = big["o_w"].astype(np.float32)   # the routing weights as a fp32 tensor carries them
    pos, ors = to_dev(opos), to_dev(big["ors"])
    wd = to_dev(w)
    q = torch.empty((R, I), dtype=torch.uint8, device=dev)
    s = torch.empty((R, I // 128), dtype=torch.float32, device=dev)
    qt = torch.empty((I, R), dtype=torch.uint8, device=dev)
    st = torch.empty((I, R // 128), dtype=torch.float32, device=dev)
    tk.tk_swiglu_quant_t(h, ors, pos, wd, q, s, qt, st)
    q2 = torch.empty_like(q)
    s2 = torch.empty_like(s)
    tk.tk_swiglu_quant(h, None, ors, pos, wd, q2, s2)
    torch.cuda.synchronize()
    row_w = oracle.row_weights(opos, w, R)
    n_blk = R // 128
    blocks = sorted({0, n_blk - 1, *big["rng"].choice(n_blk, 3, replace=False).tolist()})
    for b in blocks:
        r0, r1 = 128 * b, 128 * b + 128
        h_b = _bits(h[r0:r1])
        q_ref, s_ref = oracle.swiglu_quant(h_b, I, row_w[r0:r1])
        qt_ref, st_ref = oracle.swiglu_quant_t(h_b, I, row_w[r0:r1])
        assert np.array_equal(to_host(q[r0:r1]), q_ref), f"row-major codes, block {b}"
        assert np.array_equal(to_host(s[r0:r1]), s_ref), f"row-major scales, block {b}"
        assert np.array_equal(to_host(q2[r0:r1]), q_ref), f"plain form codes, block {b}"
        assert np.array_equal(to_host(s2[r0:r1]), s_ref), f"plain form scales, block {b}"
        assert np.array_equal(to_host(qt[:, r0:r1]), qt_ref), f"transposed codes, block {b}"
        assert np.array_equal(to_host(st[:, b:b + 1]), st_ref), f"transposed scales, block {b}"
    del h, q, s, qt, st, q2, s2
    torch.cuda.empty_cache()


@pytest.mark.parametrize("mode_name", ["TK_QUANT_FP8_1X128", "TK_QUANT_FP8_1X128_POW2",
                                       "TK_QUANT_FP8_128X128", "TK_QUANT_FP4_1X32"])
def test_large_quant_modes(big, mode_name):
    """The codec granularities whose blocks are local to a row or a 128-row
    block, over an 8.8 GB matrix (per-channel scales need every row and are
    covered at the hidden-state shape)."""
    dev, mode = big["dev"], getattr(tk, mode_name)
    x = _gpu_bf16((R, H), 14, dev)
    q, sc = tk.tk_quant(x, mode)
    torch.cuda.synchronize()
    n_blk = R // 128
    blocks = sorted({0, n_blk - 1, *big["rng"].choice(n_blk, 2, replace=False).tolist()})
    for b in blocks:
        r0, r1 = 128 * b, 128 * b + 128
        q_ref, s_ref = oracle.quant(_bits(x[r0:r1]), mode)
        assert np.array_equal(to_host(q[r0:r1]), q_ref), f"codes, block {b}"
        g_s = to_host(sc[b:b + 1]) if mode == tk.TK_QUANT_FP8_128X128 else to_host(sc[r0:r1])
        assert np.array_equal(g_s, s_ref), f"scales, block {b}"
    del x, q, sc
    torch.cuda.empty_cache()
