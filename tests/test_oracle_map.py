"""Pins of the oracle's map step: counts, offsets, stable positions, mask.

Checked against torch library routines (bincount, cumsum, stable argsort) and
the invariants of a stable expert-major permutation.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_routing_amd import synth


def _torch_map(idx: np.ndarray, lo: int, hi: int):
    T, k = idx.shape
    flat = torch.from_numpy(idx.reshape(-1).astype(np.int64))
    valid = (flat >= lo) & (flat < hi)
    counts = torch.bincount(flat[valid] - lo, minlength=hi - lo)
    offsets = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(counts, 0)])
    # stable sort of the valid flat routes by expert: token order within expert
    key = torch.where(valid, flat, torch.tensor(1 << 40))
    order = torch.sort(key, stable=True).indices[: int(valid.sum())]
    pos = torch.full((T * k,), -1, dtype=torch.int64)
    pos[order] = torch.arange(order.numel())
    row_src = order // k
    return counts.numpy(), offsets.numpy(), pos.view(T, k).numpy(), row_src.numpy()


@pytest.mark.parametrize("T,E,k,lo,hi", [
    (1, 4, 1, 0, 4), (37, 16, 2, 0, 16), (500, 64, 6, 0, 64), (1000, 256, 8, 0, 256),
    (1000, 256, 8, 32, 64), (333, 32, 4, 5, 6), (0, 8, 2, 0, 8),
])
def test_map_matches_torch(T, E, k, lo, hi):
    rng = np.random.default_rng(T + E + k + lo)
    idx = synth.random_routing(rng, T, E, k)
    counts, offsets, pos, row_src = oracle.map_routes(idx, E, lo, hi)
    c2, o2, p2, r2 = _torch_map(idx, lo, hi)
    assert np.array_equal(counts, c2)
    assert np.array_equal(offsets, o2)
    assert np.array_equal(pos, p2)
    assert np.array_equal(row_src, r2)


def test_map_invariants_v3_shape():
    rng = np.random.default_rng(20)
    T, E, k = 8192, 256, 8
    idx = synth.random_routing(rng, T, E, k)
    counts, offsets, pos, row_src = oracle.map_routes(idx, E)
    R = T * k
    assert counts.sum() == R and offsets[-1] == R and offsets[0] == 0
    assert np.array_equal(np.sort(pos.ravel()), np.arange(R))          # bijection
    assert np.array_equal(row_src[pos.ravel()], np.repeat(np.arange(T), k))
    # rows are sorted by (expert, token)
    e_of_row = np.empty(R, np.int64)
    e_of_row[pos.ravel()] = idx.ravel()
    assert np.all(np.diff(e_of_row) >= 0)
    same = np.diff(e_of_row) == 0
    assert np.all(np.diff(row_src)[same] > 0)


def test_map_mask_and_empty_experts():
    rng = np.random.default_rng(21)
    T, E, k = 400, 64, 4
    idx = synth.random_routing(rng, T, E - 1, k)
    idx = np.where(idx >= 40, idx + 1, idx).astype(np.int32)   # expert 40 never chosen
    counts, offsets, pos, row_src = oracle.map_routes(idx, E, 32, 48)
    valid = (idx >= 32) & (idx < 48)
    assert np.array_equal(pos < 0, ~valid)
    assert counts[40 - 32] == 0 and offsets[40 - 32] == offsets[41 - 32]
    assert counts.sum() == valid.sum() == offsets[-1]


def test_map_repeated_id_routed_once():
    idx = np.array([[3, 3, 1], [1, 2, 1], [0, 0, 0]], np.int32)
    counts, offsets, pos, row_src = oracle.map_routes(idx, 4)
    assert counts.tolist() == [1, 2, 1, 1]
    assert offsets.tolist() == [0, 1, 3, 4, 5]
    assert pos.tolist() == [[4, -1, 1], [2, 3, -1], [0, -1, -1]]
    assert row_src.tolist() == [2, 0, 1, 1, 0]


def _torch_map_aligned(idx: np.ndarray, lo: int, hi: int, align: int):
    """The torch reference above, with each expert's segment padded to a
    multiple of `align` rows (padding rows have no source token: -1)."""
    counts, _, pos_plain, row_src_plain = _torch_map(idx, lo, hi)
    c = torch.from_numpy(counts.astype(np.int64))
    padded = (c + align - 1) // align * align
    offsets = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(padded, 0)])
    plain_off = torch.cat([torch.zeros(1, dtype=torch.int64), torch.cumsum(c, 0)])
    T, k = idx.shape
    flat = torch.from_numpy(idx.reshape(-1).astype(np.int64))
    p = torch.from_numpy(pos_plain.reshape(-1).astype(np.int64))
    valid = p >= 0
    e = torch.where(valid, flat - lo, torch.zeros_like(flat))
    pos = torch.where(valid, p - plain_off[e] + offsets[e], torch.full_like(p, -1))
    row_src = torch.full((int(offsets[-1]),), -1, dtype=torch.int64)
    row_src[pos[valid]] = torch.arange(T * k)[valid] // k
    return counts, offsets.numpy(), pos.view(T, k).numpy(), row_src.numpy()


@pytest.mark.parametrize("T,E,k,lo,hi,align", [
    (37, 16, 2, 0, 16, 1), (500, 64, 6, 0, 64, 128), (1000, 256, 8, 0, 256, 128),
    (1000, 256, 8, 32, 64, 64), (333, 32, 4, 5, 9, 7), (0, 8, 2, 0, 8, 16), (64, 16, 2, 0, 16, 3),
])
def test_map_aligned_matches_torch(T, E, k, lo, hi, align):
    rng = np.random.default_rng(T + E + k + lo + align)
    idx = synth.random_routing(rng, T, E, k)
    got = oracle.map_aligned(idx, E, lo, hi, align)
    ref = _torch_map_aligned(idx, lo, hi, align)
    for g, r, name in zip(got, ref, ("counts", "offsets", "pos", "row_src")):
        assert np.array_equal(g, r), name
    counts, offsets, pos, row_src = got
    assert np.all(offsets % align == 0)
    assert np.all(np.diff(offsets) >= counts) and np.all(np.diff(offsets) - counts < align)
    if align == 1:
        plain = oracle.map_routes(idx, E, lo, hi)
        for g, r in zip(got, plain):
            assert np.array_equal(g, r)
