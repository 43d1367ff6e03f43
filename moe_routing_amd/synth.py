"""Seeded synthetic inputs shaped like the pages' MoE workload.

This module only draws random numbers and lays them out; it computes none of
the routing pipeline.  Both the HIP path and the CPU oracle consume what it
returns.  bf16 tensors are returned as uint16 arrays of bf16 bit patterns
(fp32 draws rounded to nearest-even by torch's cast).

Workloads (DeepSeek-V3 shape, as on "剛剛，DeepSeek開始頻繁更新：Tile Kernels、
DeepEP V2", section 性能表現: 8K tokens per batch, hidden 7168, top-8 experts;
256 experts with 8 active, "刚刚！DeepSeek开源高性能GPU算子库TileKernels",
item moe/):

  tiny          T=64,   E=16,  k=2, H=256; softmax top-2, weights renormalised;
                logits N(0,1); hidden bf16 N(0,1); expert outputs bf16 N(0,1)
                of shape (T*k, H).
  v3_gate       T=8192, E=256 (8 groups of 32), k=8; logits N(0,1); bias
                U(-0.1, 0.1) (selection only); sigmoid; top-2 group sums, top-4
                groups, weights scaled by 2.5.
  v3_expand     hidden bf16 N(0,1) of (8192, 7168), 1 % of the rows (82 rows)
                multiplied by 50 before rounding; routing of v3_gate.
  v3_combine    expert outputs bf16 N(0,1) of (65536, 7168) in expert order;
                routing of v3_gate.
  ep_share      T=32768, H=7168, E=256, k=8; logits N(0,1) plus a per-expert
                log-Zipf(s=1.2) popularity offset -1.2*ln(rank), rank a seeded
                permutation of 1..256; only experts 32..63 are local; v3 gating
                without bias; hidden bf16 N(0,1).

Each workload draws from numpy's PCG64 ``default_rng(seed)`` in the order
listed above.
"""
from __future__ import annotations

import numpy as np
import torch

SOFTMAX, SIGMOID = 0, 1


def bf16_bits(a32: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (torch cast, nearest-even); return bits."""
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float32)


def normal_bf16(rng: np.random.Generator, shape, chunk_rows: int = 8192) -> np.ndarray:
    """bf16 N(0,1) bits, drawn row block by row block to bound host memory."""
    shape = tuple(shape)
    out = np.empty(shape, np.uint16)
    rows = shape[0]
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        out[r0:r1] = bf16_bits(rng.standard_normal((r1 - r0,) + shape[1:], dtype=np.float32))
    return out


# Routing options of each workload (score, n_groups, topk_groups, group_topn,
# renormalize, route_scale).
ROUTE_TINY = dict(score=SOFTMAX, n_groups=1, topk_groups=1, group_topn=0,
                  renormalize=1, route_scale=1.0)
ROUTE_V3 = dict(score=SIGMOID, n_groups=8, topk_groups=4, group_topn=2,
                renormalize=1, route_scale=2.5)


def tiny(seed: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    T, E, k, H = 64, 16, 2, 256
    logits = normal_f32(rng, (T, E))
    x = normal_bf16(rng, (T, H))
    y = normal_bf16(rng, (T * k, H))
    return dict(name="tiny", T=T, E=E, k=k, H=H, logits=logits, bias=None, x=x, y=y,
                local=(0, E), route=dict(ROUTE_TINY))


def v3_gate(seed: int = 0, T: int = 8192) -> dict:
    rng = np.random.default_rng(seed)
    E, k = 256, 8
    logits = normal_f32(rng, (T, E))
    bias = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    return dict(name="v3_gate", T=T, E=E, k=k, logits=logits, bias=bias,
                local=(0, E), route=dict(ROUTE_V3))


def v3_hidden(seed: int = 0, T: int = 8192, H: int = 7168,
              outlier_frac: float = 0.01, outlier_mult: float = 50.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    z = normal_f32(rng, (T, H))
    n_out = int(np.ceil(outlier_frac * T))
    rows = rng.choice(T, size=n_out, replace=False)
    z[rows] *= np.float32(outlier_mult)
    return bf16_bits(z)


def v3_expert_out(seed: int = 0, R: int = 65536, H: int = 7168) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return normal_bf16(rng, (R, H))


def ep_share(seed: int = 0, T: int = 32768, H: int = 7168) -> dict:
    rng = np.random.default_rng(seed)
    E, k = 256, 8
    z = normal_f32(rng, (T, E))
    rank = rng.permutation(E) + 1
    offset = (-1.2 * np.log(rank.astype(np.float64))).astype(np.float32)
    logits = (z + offset[None, :]).astype(np.float32)
    x = normal_bf16(rng, (T, H))
    return dict(name="ep_share", T=T, E=E, k=k, H=H, logits=logits, bias=None, x=x,
                local=(32, 64), route=dict(ROUTE_V3, ), zipf_rank=rank)


def random_routing(rng: np.random.Generator, T: int, E: int, k: int) -> np.ndarray:
    """k distinct experts per token, uniformly at random (for unit tests of map)."""
    keys = rng.random((T, E))
    return np.argsort(keys, axis=1)[:, :k].astype(np.int32)
