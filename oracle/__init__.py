"""ctypes wrapper of the plain C oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package.  The product path
(``moe_routing_amd``) never imports it and never falls back to it.

Every function takes and returns numpy arrays; bf16 tensors are uint16 arrays
holding the bf16 bit patterns, FP8 tensors are uint8 arrays of E4M3 codes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# Every fp32 operation in oracle.c must be one IEEE-rounded operation.
GCC_CMD = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]

SOFTMAX, SIGMOID = 0, 1

_lib = None


def build() -> str:
    """Compile liboracle.so from oracle.c (always recompiles)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _declare(ctypes.CDLL(_LIB))
    return _lib


def _p(a: np.ndarray | None):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _declare(L: ctypes.CDLL) -> ctypes.CDLL:
    vp, i32, i64, f32, f64 = (ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                              ctypes.c_float, ctypes.c_double)
    L.orc_route.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, f64, vp, vp]
    L.orc_route.restype = i32
    L.orc_map.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.orc_map.restype = i32
    L.orc_map_aligned.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp]
    L.orc_map_aligned.restype = i32
    L.orc_balance_loss.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp]
    L.orc_balance_loss.restype = i32
    L.orc_pow2_scale_e4m3.argtypes = [f32]
    L.orc_pow2_scale_e4m3.restype = f32
    L.orc_quant_1x128.argtypes = [vp, i64, i32, i32, vp, vp]
    L.orc_quant_1x128.restype = None
    L.orc_quant_128x128.argtypes = [vp, i64, i32, vp, vp]
    L.orc_quant_128x128.restype = None
    L.orc_quant_per_channel.argtypes = [vp, i64, i32, vp, vp]
    L.orc_quant_per_channel.restype = None
    L.orc_quant_fp4_1x32.argtypes = [vp, i64, i32, vp, vp]
    L.orc_quant_fp4_1x32.restype = None
    L.orc_e2m1_to_f64.argtypes = [ctypes.c_uint8]
    L.orc_e2m1_to_f64.restype = f64
    L.orc_e2m1_from_f32_n.argtypes = [vp, i64, vp]
    L.orc_e2m1_from_f32_n.restype = None
    L.orc_expand.argtypes = [vp, i32, i32, i32, vp, i32, i64, vp, vp]
    L.orc_expand.restype = i32
    L.orc_quant_row.argtypes = [vp, i32, vp, vp]
    L.orc_quant_row.restype = None
    L.orc_standin.argtypes = [vp, vp, i64, i32, f32, vp]
    L.orc_standin.restype = None
    L.orc_reduce.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp]
    L.orc_reduce.restype = i32
    L.orc_quant_f32_row.argtypes = [vp, i32, vp, vp]
    L.orc_quant_f32_row.restype = None
    L.orc_row_weights.argtypes = [vp, vp, i32, i32, i64, vp]
    L.orc_row_weights.restype = None
    L.orc_swiglu_quant.argtypes = [vp, i64, i32, vp, vp, vp]
    L.orc_swiglu_quant.restype = i32
    L.orc_swiglu_f32.argtypes = [vp, i64, i32, vp, vp]
    L.orc_swiglu_f32.restype = i32
    L.orc_swiglu_quant_t.argtypes = [vp, i64, i32, vp, vp, vp]
    L.orc_swiglu_quant_t.restype = i32
    for name in ("orc_e4m3_from_f32_n", "orc_bf16_from_f32_n", "orc_bf16_from_f64_n",
                 "orc_sigmoid_f32_n", "orc_exp_f32_n"):
        getattr(L, name).argtypes = [vp, i64, vp]
        getattr(L, name).restype = None
    L.orc_e4m3_to_f64.argtypes = [ctypes.c_uint8]
    L.orc_e4m3_to_f64.restype = f64
    L.orc_route_key.argtypes = [f32, i32, vp, i32]
    L.orc_route_key.restype = f32
    return L


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- codecs ----
def e4m3_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    lib().orc_e4m3_from_f32_n(_p(v), v.size, _p(q))
    return q


def e4m3_to_f64(q) -> np.ndarray:
    q = _c(q, np.uint8)
    f = lib().orc_e4m3_to_f64
    table = np.array([f(c) for c in range(256)], np.float64)
    return table[q]


def bf16_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    h = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_f32_n(_p(v), v.size, _p(h))
    return h


def bf16_from_f64(v) -> np.ndarray:
    v = _c(v, np.float64)
    h = np.empty(v.shape, np.uint16)
    lib().orc_bf16_from_f64_n(_p(v), v.size, _p(h))
    return h


def bf16_to_f32(h) -> np.ndarray:
    h = _c(h, np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def sigmoid_f32(x) -> np.ndarray:
    x = _c(x, np.float32)
    s = np.empty(x.shape, np.float32)
    lib().orc_sigmoid_f32_n(_p(x), x.size, _p(s))
    return s


def exp_f32(x) -> np.ndarray:
    x = _c(x, np.float32)
    s = np.empty(x.shape, np.float32)
    lib().orc_exp_f32_n(_p(x), x.size, _p(s))
    return s


def route_keys(logits, score: int, bias=None) -> np.ndarray:
    """Selection keys the oracle ranks on (fp32), shape of logits."""
    logits = _c(logits, np.float32)
    if score == SOFTMAX:
        return logits.copy()
    s = sigmoid_f32(logits)
    if bias is not None:
        s = (s + _c(bias, np.float32)).astype(np.float32)  # fp32 add, RN
    return s


# ----------------------------------------------------------------- steps ----
def route(logits, bias, k: int, score: int, n_groups: int = 1, topk_groups: int = 1,
          group_topn: int = 0, renormalize: int = 1, route_scale: float = 1.0):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    b = None if bias is None else _c(bias, np.float32)
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    rc = lib().orc_route(_p(logits), _p(b), T, E, k, score, n_groups, topk_groups,
                         group_topn, renormalize, float(route_scale), _p(idx), _p(w))
    if rc != 0:
        raise ValueError("oracle route: unsupported arguments")
    return idx, w


def map_routes(topk_idx, E: int, lo: int = 0, hi: int | None = None, with_row_src=True):
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    hi = E if hi is None else hi
    nl = hi - lo
    counts = np.empty(nl, np.int32)
    offsets = np.empty(nl + 1, np.int32)
    pos = np.empty((T, k), np.int32)
    row_src = np.full(T * k, -1, np.int32) if with_row_src else None
    rc = lib().orc_map(_p(topk_idx), T, k, E, lo, hi, _p(counts), _p(offsets), _p(pos),
                       _p(row_src))
    if rc != 0:
        raise ValueError("oracle map: unsupported arguments")
    if with_row_src:
        row_src = row_src[: int(offsets[-1])].copy()
    return counts, offsets, pos, row_src


def balance_loss(logits, topk_idx, score: int):
    """(f, P, loss): per-expert load fraction E/(kT)*count, mean normalised
    score, and sum_e f_e P_e (fp64)."""
    logits = _c(logits, np.float32)
    topk_idx = _c(topk_idx, np.int32)
    T, E = logits.shape
    k = topk_idx.shape[1]
    f = np.empty(E, np.float64)
    P = np.empty(E, np.float64)
    loss = np.empty(1, np.float64)
    if lib().orc_balance_loss(_p(logits), T, E, k, score, _p(topk_idx), _p(f), _p(P), _p(loss)) != 0:
        raise ValueError("oracle balance_loss: unsupported arguments")
    return f, P, float(loss[0])


def map_aligned(topk_idx, E: int, lo: int = 0, hi: int | None = None, align: int = 1):
    """Map with expert segments padded to multiples of `align` rows; row_src
    covers all offsets[-1] rows, -1 on padding rows."""
    topk_idx = _c(topk_idx, np.int32)
    T, k = topk_idx.shape
    hi = E if hi is None else hi
    nl = hi - lo
    counts = np.empty(nl, np.int32)
    offsets = np.empty(nl + 1, np.int32)
    pos = np.empty((T, k), np.int32)
    row_src = np.empty(T * k + nl * (align - 1), np.int32)
    rc = lib().orc_map_aligned(_p(topk_idx), T, k, E, lo, hi, align, _p(counts), _p(offsets),
                               _p(pos), _p(row_src))
    if rc != 0:
        raise ValueError("oracle map_aligned: unsupported arguments")
    return counts, offsets, pos, row_src[: int(offsets[-1])].copy()


def quant_row(x_row):
    """1x128 E4M3 quantisation of one or more bf16 rows (uint16, (..., H))."""
    x = _c(x_row, np.uint16)
    H = x.shape[-1]
    flat = x.reshape(-1, H)
    q = np.empty(flat.shape, np.uint8)
    sc = np.empty((flat.shape[0], H // 128), np.float32)
    for i in range(flat.shape[0]):
        lib().orc_quant_row(_p(flat[i]), H, _p(q[i]), _p(sc[i]))
    return q.reshape(x.shape), sc.reshape(x.shape[:-1] + (H // 128,))


def expand(x, pos, mode: int, rows_capacity: int):
    x = _c(x, np.uint16)
    pos = _c(pos, np.int32)
    T, H = x.shape
    k = pos.shape[1]
    if mode == 0:
        out = np.zeros((rows_capacity, H), np.uint16)
        scales = None
    else:
        out = np.zeros((rows_capacity, H), np.uint8)
        scales = np.zeros((rows_capacity, H // 128), np.float32)
    rc = lib().orc_expand(_p(x), T, H, k, _p(pos), mode, rows_capacity, _p(out), _p(scales))
    if rc != 0:
        raise ValueError("oracle expand: unsupported arguments")
    return out, scales


def standin(xq, scales, mult: float = 0.5):
    xq = _c(xq, np.uint8)
    scales = _c(scales, np.float32)
    R, H = xq.shape
    y = np.empty((R, H), np.uint16)
    lib().orc_standin(_p(xq), _p(scales), R, H, float(mult), _p(y))
    return y


def reduce(y, pos, w):
    y = _c(y, np.uint16)
    pos = _c(pos, np.int32)
    w = _c(w, np.float32)
    T, k = pos.shape
    R, H = y.shape
    out = np.empty((T, H), np.uint16)
    rc = lib().orc_reduce(_p(y), R, _p(pos), _p(w), T, k, H, _p(out))
    if rc != 0:
        raise ValueError("oracle reduce: unsupported arguments")
    return out


# ------------------------------------------------------- next: SwiGLU + FP8 --
def quant_f32_row(a):
    """1x128 E4M3 quantisation of fp32 rows ((..., n), n % 128 == 0)."""
    a = _c(a, np.float32)
    n = a.shape[-1]
    flat = a.reshape(-1, n)
    q = np.empty(flat.shape, np.uint8)
    sc = np.empty((flat.shape[0], n // 128), np.float32)
    for i in range(flat.shape[0]):
        lib().orc_quant_f32_row(_p(flat[i]), n, _p(q[i]), _p(sc[i]))
    return q.reshape(a.shape), sc.reshape(a.shape[:-1] + (n // 128,))


def row_weights(pos, w, rows: int):
    pos = _c(pos, np.int32)
    w = _c(w, np.float32)
    T, k = pos.shape
    out = np.empty(rows, np.float32)
    lib().orc_row_weights(_p(pos), _p(w), T, k, rows, _p(out))
    return out


def swiglu_f32(h, I: int, row_w=None):
    h = _c(h, np.uint16)
    rows = h.shape[0]
    a = np.empty((rows, I), np.float32)
    rw = None if row_w is None else _c(row_w, np.float32)
    if lib().orc_swiglu_f32(_p(h), rows, I, _p(rw), _p(a)) != 0:
        raise ValueError("oracle swiglu: unsupported arguments")
    return a


def swiglu_quant_t(h, I: int, row_w=None):
    """Transposed output: a^T (I, rows) with 1x128 blocks along its rows."""
    h = _c(h, np.uint16)
    rows = h.shape[0]
    q = np.empty((I, rows), np.uint8)
    sc = np.empty((I, rows // 128), np.float32)
    rw = None if row_w is None else _c(row_w, np.float32)
    if lib().orc_swiglu_quant_t(_p(h), rows, I, _p(rw), _p(q), _p(sc)) != 0:
        raise ValueError("oracle swiglu_quant_t: unsupported arguments")
    return q, sc


def swiglu_quant(h, I: int, row_w=None):
    h = _c(h, np.uint16)
    rows = h.shape[0]
    q = np.empty((rows, I), np.uint8)
    sc = np.empty((rows, I // 128), np.float32)
    rw = None if row_w is None else _c(row_w, np.float32)
    if lib().orc_swiglu_quant(_p(h), rows, I, _p(rw), _p(q), _p(sc)) != 0:
        raise ValueError("oracle swiglu_quant: unsupported arguments")
    return q, sc


# ------------------------------------------------ next: quant granularities --
QUANT_FP8_1X128, QUANT_FP8_1X128_POW2, QUANT_FP8_128X128, QUANT_FP8_PER_CHANNEL, QUANT_FP4_1X32 = range(5)


def quant(x, mode: int):
    """Quantise a bf16 matrix (uint16 bits, (rows, cols)); returns (codes, scales)."""
    x = _c(x, np.uint16)
    rows, cols = x.shape
    L = lib()
    if mode in (QUANT_FP8_1X128, QUANT_FP8_1X128_POW2):
        q = np.empty((rows, cols), np.uint8)
        sc = np.empty((rows, cols // 128), np.float32)
        L.orc_quant_1x128(_p(x), rows, cols, int(mode == QUANT_FP8_1X128_POW2), _p(q), _p(sc))
    elif mode == QUANT_FP8_128X128:
        q = np.empty((rows, cols), np.uint8)
        sc = np.empty(((rows + 127) // 128, cols // 128), np.float32)
        L.orc_quant_128x128(_p(x), rows, cols, _p(q), _p(sc))
    elif mode == QUANT_FP8_PER_CHANNEL:
        q = np.empty((rows, cols), np.uint8)
        sc = np.empty(cols, np.float32)
        L.orc_quant_per_channel(_p(x), rows, cols, _p(q), _p(sc))
    elif mode == QUANT_FP4_1X32:
        q = np.empty((rows, cols // 2), np.uint8)
        sc = np.empty((rows, cols // 32), np.float32)
        L.orc_quant_fp4_1x32(_p(x), rows, cols, _p(q), _p(sc))
    else:
        raise ValueError(f"unknown quant mode {mode}")
    return q, sc


def pow2_scale_e4m3(amax: float) -> float:
    return float(lib().orc_pow2_scale_e4m3(float(amax)))


def e2m1_from_f32(v) -> np.ndarray:
    v = _c(v, np.float32)
    q = np.empty(v.shape, np.uint8)
    lib().orc_e2m1_from_f32_n(_p(v), v.size, _p(q))
    return q


def e2m1_to_f64(q) -> np.ndarray:
    q = _c(q, np.uint8)
    table = np.array([lib().orc_e2m1_to_f64(c) for c in range(16)], np.float64)
    return table[q & 15]
