"""Wide rows: the expand and both combines at hidden sizes far above the
DeepSeek-V3 width, where each wave walks many chunks of a row and the dense
combine's workgroups hold few tokens.

H = 16384 and 32768 (the staged combine holds at most 7 and 3 tokens per
workgroup; here 4 and 2, two rounds), 114688 (the widest row the staged form
takes: one token per workgroup) and 114696 (bf16 only, not a multiple of 128:
a partly filled last unit, and tk_reduce_dense falls back to the
one-wave-per-unit kernel).  Routings are
dense (every slot has a row, expert-contiguous as tk_map lays them out) with
a few slots masked.  FP8 codes, scales and bf16 rows are compared with the
oracle in full; the combines on sampled tokens (first, last, random), and
tk_reduce_dense must equal tk_reduce bit for bit everywhere.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import combine_report, to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


@pytest.mark.parametrize("T,k,H", [(2000, 4, 16384), (800, 2, 32768), (300, 2, 114688),
                                   (280, 2, 114696)])
def test_wide_rows_expand_and_combine(T, k, H):
    rng = np.random.default_rng(H + T)
    E = 64
    idx = synth.random_routing(rng, T, E, k)
    _, _, pos, _ = oracle.map_routes(idx, E)
    pos = pos.copy()
    pos[rng.random((T, k)) < 0.05] = -1
    R = T * k
    x = synth.normal_bf16(rng, (T, H))
    xd, pd = to_dev(x, bf16=True), to_dev(pos)

    xe, _ = tk.tk_expand_quant(xd, pd, tk.TK_EXPAND_BF16, R)
    o_xe, _ = oracle.expand(x, pos, 0, R)
    valid = np.zeros(R, bool)
    valid[pos[pos >= 0]] = True
    assert np.array_equal(to_host(xe)[valid], o_xe[valid]), "bf16 rows"
    del xe
    if H % 128 == 0:
        xq, sc = tk.tk_expand_quant(xd, pd, tk.TK_EXPAND_FP8_E4M3_1X128, R)
        o_xq, o_sc = oracle.expand(x, pos, 1, R)
        assert np.array_equal(to_host(xq)[valid], o_xq[valid]), "FP8 codes"
        assert np.array_equal(to_host(sc)[valid], o_sc[valid]), "scales"
        del xq, sc

    dev = xd.device
    g = torch.Generator(device=dev)
    g.manual_seed(H)
    y = torch.randn((R, H), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    w = rng.uniform(0.05, 0.6, (T, k)).astype(np.float32)
    wd = to_dev(w)
    dense = tk.tk_reduce_dense(y, pd, wd)
    plain = tk.tk_reduce(y, pd, wd)
    torch.cuda.synchronize()
    assert torch.equal(dense, plain), "tk_reduce_dense differs from tk_reduce"
    sample = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 24, replace=False)]))
    rows = pos[sample]
    used = rows[rows >= 0]
    y_s = to_host(y[torch.from_numpy(used.astype(np.int64)).to(dev)])
    pos_s = np.full(rows.shape, -1, np.int32)
    pos_s[rows >= 0] = np.arange(used.size, dtype=np.int32)
    rep = combine_report(to_host(dense[torch.from_numpy(sample).to(dev)]),
                         oracle.reduce(y_s, pos_s, w[sample]))
    assert rep["ok"], rep
