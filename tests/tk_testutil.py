"""Helpers for the GPU parity tests: host<->device moves of numpy arrays that
hold bf16 bit patterns, and the combine tolerance."""
import numpy as np
import torch

import oracle


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, bf16: bool = False) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if bf16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


# Combine tolerance: |gpu - ref| <= 1e-2 + 1e-2 * |ref| per element, in bf16.
COMBINE_ATOL = 1e-2
COMBINE_RTOL = 1e-2
# Weights: fp32 evaluation (sigmoid within 3 ulp, sequential slot-order sum of
# <= 32 terms, one division, one scaling) against fp64: well inside 4e-6 rel.
W_RTOL = 4e-6
W_ATOL = 1e-9


def combine_report(got_bits: np.ndarray, ref_bits: np.ndarray) -> dict:
    g = oracle.bf16_to_f32(got_bits).astype(np.float64)
    r = oracle.bf16_to_f32(ref_bits).astype(np.float64)
    err = np.abs(g - r)
    ok = err <= COMBINE_ATOL + COMBINE_RTOL * np.abs(r)
    return dict(ok=bool(ok.all()), max_abs=float(err.max(initial=0.0)),
                max_rel=float((err / np.maximum(np.abs(r), 1e-30)).max(initial=0.0)),
                bit_exact_frac=float((got_bits == ref_bits).mean()) if got_bits.size else 1.0,
                n_bad=int((~ok).sum()))


def route_kwargs(cfg: dict) -> dict:
    return dict(cfg["route"])
