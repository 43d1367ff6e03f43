"""tk_map_noalloc on the GPU: the map with its count matrix in the library's
per-GPU scratch array, called through the C ABI, against tk_map with a
caller-provided workspace -- bit-exact, on two calls in a row, the second
with a smaller input (and a local-expert mask), so that the second reuses
the array the first left behind."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth
from tk_testutil import to_dev, to_host

pytestmark = pytest.mark.gpu

tk = pytest.importorskip("moe_routing_amd")


def _noalloc(idx, E, lo, hi):
    L = tk.library()
    T, k = idx.shape
    nl = hi - lo
    dev = idx.device
    counts = torch.full((nl,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((nl + 1,), -7, dtype=torch.int32, device=dev)
    pos = torch.full((T, k), -7, dtype=torch.int32, device=dev)
    row_src = torch.full((T * k,), -7, dtype=torch.int32, device=dev)
    st = L.tk_map_noalloc(ctypes.c_void_p(idx.data_ptr()), T, k, E, lo, hi,
                          ctypes.c_void_p(counts.data_ptr()), ctypes.c_void_p(offsets.data_ptr()),
                          ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(row_src.data_ptr()),
                          ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, L.tk_last_error()
    return counts, offsets, pos, row_src


def test_map_noalloc_matches_map_twice():
    # both calls run the count pass into the scratch array: the first through
    # the separate scan (T=40000, 256 experts: more than 32768 counts), the
    # second, smaller one with a local-expert mask summing the per-tile counts
    # in the place pass
    rng = np.random.default_rng(5)
    cases = [(synth.random_routing(rng, 40000, 256, 8), 256, 0, 256),
             (synth.random_routing(rng, 33000, 64, 8), 64, 16, 48)]
    for idx_h, E, lo, hi in cases:
        idx = to_dev(idx_h)
        got = _noalloc(idx, E, lo, hi)
        ref = tk.tk_map(idx, E, lo, hi)
        torch.cuda.synchronize()
        R = int(to_host(ref[1])[-1])
        assert np.array_equal(to_host(got[0]), to_host(ref[0]))
        assert np.array_equal(to_host(got[1]), to_host(ref[1]))
        assert np.array_equal(to_host(got[2]), to_host(ref[2]))
        assert np.array_equal(to_host(got[3])[:R], to_host(ref[3])[:R])
        # and both equal the oracle's map
        oc, oo, op, ors = oracle.map_routes(idx_h, E, lo, hi)
        assert np.array_equal(to_host(got[2]), op) and np.array_equal(to_host(got[3])[:R], ors)
