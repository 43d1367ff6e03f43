"""MI355X (gfx950) MoE routing hot path: thin ctypes binding of libtk.so.

The functions below carry the names of the C entry points declared in
include/tk.h and only marshal arguments: they check dtypes, devices and
shapes of torch tensors, allocate outputs the caller did not pass, and hand
raw device pointers plus torch's current HIP stream to the library.  Every
step of the path runs in the library's HIP kernels; there is no fallback.

    tk_route(logits, bias, k, opts)            -> (topk_idx, topk_w)
    tk_map(topk_idx, E, local_begin, local_end) -> (counts, offsets, pos, row_src)
    tk_map_aligned(topk_idx, E, local_begin, local_end, align) -> (counts, offsets, pos, row_src)
    tk_map_noalloc(topk_idx, E, local_begin, local_end) -> tk_map without a workspace
    tk_expand_quant(x, pos, mode, rows_capacity) -> (out, scales)
    tk_reduce(y, pos, topk_w)                  -> out
    tk_reduce_dense(y, pos, topk_w)            -> out (the same, dense routings)
    tk_expert_standin(xq, scales, n_rows, mult) -> y
    tk_swiglu_quant(h, I, n_rows, row_src, pos, topk_w) -> (out, scales)
    tk_swiglu_quant_t(h, row_src, pos, topk_w) -> (out, scales, out_t, scales_t)
    tk_silu_bf16(g) -> fp32 RN(g * sigmoid(g))
    tk_balance_loss(logits, topk_idx, score)   -> (f, P, loss)
    tk_quant(x, mode)                          -> (codes, scales)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtk.so")

TK_OK, TK_ERR_ARG, TK_ERR_UNSUPPORTED, TK_ERR_DEVICE = 0, -1, -2, -3
TK_MAX_EXPERTS, TK_MAX_TOPK = 1024, 32
TK_MAP_NOALLOC_SCRATCH_BYTES = 1 << 20
TK_SCORE_SOFTMAX, TK_SCORE_SIGMOID = 0, 1
TK_EXPAND_BF16, TK_EXPAND_FP8_E4M3_1X128 = 0, 1
(TK_QUANT_FP8_1X128, TK_QUANT_FP8_1X128_POW2, TK_QUANT_FP8_128X128, TK_QUANT_FP8_PER_CHANNEL,
 TK_QUANT_FP4_1X32) = range(5)


class TkError(RuntimeError):
    """A tk_* call returned a non-zero status."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed with status {status}: {text}")
        self.status = status


class _RouteOpts(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("route_scale", ctypes.c_float)]


@dataclass
class RouteOpts:
    score: int = TK_SCORE_SOFTMAX
    n_groups: int = 1
    topk_groups: int = 1
    group_topn: int = 0
    renormalize: int = 1
    route_scale: float = 1.0

    def _c(self) -> _RouteOpts:
        return _RouteOpts(self.score, self.n_groups, self.topk_groups, self.group_topn,
                          self.renormalize, self.route_scale)


_lib = None


def library() -> ctypes.CDLL:
    """Load libtk.so (built in-tree by __graft_entry__.build()); fail loudly if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                              "(hipcc --offload-arch=gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                 ctypes.c_float, ctypes.c_size_t)
        L.tk_last_error.argtypes = []
        L.tk_last_error.restype = ctypes.c_char_p
        L.tk_route.argtypes = [vp, vp, i32, i32, i32, ctypes.POINTER(_RouteOpts), vp, vp, vp]
        L.tk_route.restype = i32
        L.tk_map_workspace_bytes.argtypes = [i32, i32, i32]
        L.tk_map_workspace_bytes.restype = sz
        L.tk_map.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.tk_map.restype = i32
        L.tk_map_aligned.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.tk_map_aligned.restype = i32
        L.tk_map_noalloc.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.tk_map_noalloc.restype = i32
        L.tk_expand_quant.argtypes = [vp, i32, i32, i32, vp, i32, vp, vp, i64, vp]
        L.tk_expand_quant.restype = i32
        L.tk_reduce.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp]
        L.tk_reduce.restype = i32
        L.tk_reduce_dense.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp]
        L.tk_reduce_dense.restype = i32
        L.tk_expert_standin.argtypes = [vp, vp, vp, i64, i32, f32, vp, vp]
        L.tk_expert_standin.restype = i32
        L.tk_swiglu_quant.argtypes = [vp, i64, vp, i32, vp, vp, vp, i32, i32, vp, vp, vp]
        L.tk_swiglu_quant.restype = i32
        L.tk_swiglu_quant_t.argtypes = [vp, i64, i32, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp]
        L.tk_swiglu_quant_t.restype = i32
        L.tk_silu_bf16.argtypes = [vp, i64, vp, vp]
        L.tk_silu_bf16.restype = i32
        L.tk_balance_workspace_bytes.argtypes = [i32, i32]
        L.tk_balance_workspace_bytes.restype = sz
        L.tk_balance_loss.argtypes = [vp, vp, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.tk_balance_loss.restype = i32
        L.tk_quant_workspace_bytes.argtypes = [i64, i32, i32]
        L.tk_quant_workspace_bytes.restype = sz
        L.tk_quant.argtypes = [vp, i64, i32, i32, vp, vp, vp, sz, vp]
        L.tk_quant.restype = i32
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != TK_OK:
        raise TkError(fn, status, library().tk_last_error().decode())


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int | None = None,
         numel: int | None = None, device: torch.device | None = None):
    """Check a tensor handed to the library: a contiguous HIP tensor of `dtype`,
    with at least `numel` elements (the extent the C call reads or writes; the
    library cannot see tensor sizes) on `device`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other tensors on {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call needs {numel}")
    return t


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def tk_route(logits: torch.Tensor, bias: torch.Tensor | None, k: int, opts: RouteOpts,
             topk_idx: torch.Tensor | None = None, topk_w: torch.Tensor | None = None):
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    if bias is not None:
        _dev(bias, "bias", torch.float32, 1, E, dev)
    if topk_idx is None:
        topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _dev(topk_idx, "topk_idx", torch.int32, numel=T * k, device=dev)
    _dev(topk_w, "topk_w", torch.float32, numel=T * k, device=dev)
    c = opts._c()
    _check("tk_route", library().tk_route(_ptr(logits), _ptr(bias), T, E, k, ctypes.byref(c),
                                          _ptr(topk_idx), _ptr(topk_w), _stream(logits)))
    return topk_idx, topk_w


def tk_map_workspace_bytes(T: int, k: int, n_local: int) -> int:
    return int(library().tk_map_workspace_bytes(T, k, n_local))


def tk_map(topk_idx: torch.Tensor, E: int, local_begin: int = 0, local_end: int | None = None,
           counts=None, offsets=None, pos=None, row_src=None, workspace=None,
           want_row_src: bool = True):
    return tk_map_aligned(topk_idx, E, local_begin, local_end, 1, counts, offsets, pos, row_src,
                          workspace, want_row_src)


def tk_map_noalloc(topk_idx: torch.Tensor, E: int, local_begin: int = 0,
                   local_end: int | None = None, counts=None, offsets=None, pos=None,
                   row_src=None):
    """tk_map without a workspace: the count matrix lives in the library's
    per-GPU array of TK_MAP_NOALLOC_SCRATCH_BYTES.  Outputs the caller does
    not pass are allocated here (the C call itself allocates nothing)."""
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    local_end = E if local_end is None else local_end
    nl = local_end - local_begin
    dev = topk_idx.device
    counts = torch.empty(max(nl, 0), dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(max(nl, 0) + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    pos = torch.empty((T, k), dtype=torch.int32, device=dev) if pos is None else pos
    for name, t, n in (("counts", counts, max(nl, 0)), ("offsets", offsets, max(nl, 0) + 1),
                       ("pos", pos, T * k)):
        _dev(t, name, torch.int32, numel=n, device=dev)
    if row_src is not None:
        _dev(row_src, "row_src", torch.int32, numel=T * k, device=dev)
    _check("tk_map_noalloc", library().tk_map_noalloc(
        _ptr(topk_idx), T, k, E, local_begin, local_end, _ptr(counts), _ptr(offsets),
        _ptr(pos), _ptr(row_src), _stream(topk_idx)))
    return counts, offsets, pos, row_src


def tk_map_aligned(topk_idx: torch.Tensor, E: int, local_begin: int = 0,
                   local_end: int | None = None, align: int = 1, counts=None, offsets=None,
                   pos=None, row_src=None, workspace=None, want_row_src: bool = True):
    """Map with each expert's segment padded to a multiple of `align` rows.
    row_src (when allocated here) holds T*k + n_local*(align-1) entries, the
    largest padded row count."""
    _dev(topk_idx, "topk_idx", torch.int32, 2)
    T, k = topk_idx.shape
    local_end = E if local_end is None else local_end
    nl = local_end - local_begin
    dev = topk_idx.device
    counts = torch.empty(max(nl, 0), dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(max(nl, 0) + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    pos = torch.empty((T, k), dtype=torch.int32, device=dev) if pos is None else pos
    if row_src is None and want_row_src:
        row_src = torch.empty(T * k + max(nl, 0) * max(align - 1, 0), dtype=torch.int32, device=dev)
    need = tk_map_workspace_bytes(T, k, nl) if nl > 0 else 0
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    for name, t, n in (("counts", counts, max(nl, 0)), ("offsets", offsets, max(nl, 0) + 1),
                       ("pos", pos, T * k)):
        _dev(t, name, torch.int32, numel=n, device=dev)
    if row_src is not None:   # up to T*k rows plus each local segment's padding
        _dev(row_src, "row_src", torch.int32, numel=T * k + max(nl, 0) * max(align - 1, 0),
             device=dev)
    _dev(workspace, "workspace", torch.uint8, device=dev)
    _check("tk_map", library().tk_map_aligned(
        _ptr(topk_idx), T, k, E, local_begin, local_end, align, _ptr(counts), _ptr(offsets),
        _ptr(pos), _ptr(row_src), _ptr(workspace), workspace.numel(), _stream(topk_idx)))
    return counts, offsets, pos, row_src


def tk_expand_quant(x: torch.Tensor, pos: torch.Tensor, mode: int, rows_capacity: int,
                    out: torch.Tensor | None = None, scales: torch.Tensor | None = None):
    _dev(x, "x", torch.bfloat16, 2)
    T, H = x.shape
    dev = x.device
    _dev(pos, "pos", torch.int32, 2, device=dev)
    k = pos.shape[1]
    if pos.shape[0] != T:
        raise ValueError("pos must have one row per token")
    if mode == TK_EXPAND_FP8_E4M3_1X128:
        if out is None:
            out = torch.empty((rows_capacity, H), dtype=torch.uint8, device=dev)
        if scales is None:
            scales = torch.empty((rows_capacity, max(H // 128, 1)), dtype=torch.float32, device=dev)
        _dev(out, "out", torch.uint8, numel=rows_capacity * H, device=dev)
        _dev(scales, "scales", torch.float32, numel=rows_capacity * (H // 128), device=dev)
    else:
        if out is None:
            out = torch.empty((rows_capacity, H), dtype=torch.bfloat16, device=dev)
        _dev(out, "out", torch.bfloat16, numel=rows_capacity * H, device=dev)
    _check("tk_expand_quant", library().tk_expand_quant(
        _ptr(x), T, H, k, _ptr(pos), mode, _ptr(out), _ptr(scales), rows_capacity, _stream(x)))
    return out, scales


def tk_reduce(y: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor,
              out: torch.Tensor | None = None):
    return _reduce("tk_reduce", y, pos, topk_w, out)


def tk_reduce_dense(y: torch.Tensor, pos: torch.Tensor, topk_w: torch.Tensor,
                    out: torch.Tensor | None = None):
    """tk_reduce for routings where (nearly) every slot has a row: the same
    results, one burst of output rows per few tokens."""
    return _reduce("tk_reduce_dense", y, pos, topk_w, out)


def _reduce(fn: str, y, pos, topk_w, out):
    _dev(y, "y", torch.bfloat16, 2)
    dev = y.device
    _dev(pos, "pos", torch.int32, 2, device=dev)
    _dev(topk_w, "topk_w", torch.float32, 2, device=dev)
    T, k = pos.shape
    R, H = y.shape
    if tuple(topk_w.shape) != (T, k):
        raise ValueError("topk_w must match pos")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dev(out, "out", torch.bfloat16, 2, T * H, dev)
    _check(fn, getattr(library(), fn)(_ptr(y), R, _ptr(pos), _ptr(topk_w), T, k, H, _ptr(out),
                                      _stream(y)))
    return out


def tk_expert_standin(xq: torch.Tensor, scales: torch.Tensor, n_rows: torch.Tensor,
                      mult: float = 0.5, y: torch.Tensor | None = None):
    _dev(xq, "xq", torch.uint8, 2)
    cap, H = xq.shape
    dev = xq.device
    _dev(scales, "scales", torch.float32, 2, cap * (H // 128), dev)
    _dev(n_rows, "n_rows", torch.int32, numel=1, device=dev)
    if y is None:
        y = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    _dev(y, "y", torch.bfloat16, 2, cap * H, dev)
    _check("tk_expert_standin", library().tk_expert_standin(
        _ptr(xq), _ptr(scales), _ptr(n_rows), cap, H, float(mult), _ptr(y), _stream(xq)))
    return y


def tk_swiglu_quant(h: torch.Tensor, n_rows: torch.Tensor | None = None,
                    row_src: torch.Tensor | None = None, pos: torch.Tensor | None = None,
                    topk_w: torch.Tensor | None = None, out: torch.Tensor | None = None,
                    scales: torch.Tensor | None = None):
    """SwiGLU (gate = first half of each row, up = second half) fused with
    1x128 FP8 E4M3 quantisation; weighted by the routing weights when
    row_src, pos and topk_w are given."""
    _dev(h, "h", torch.bfloat16, 2)
    cap, two_i = h.shape
    if two_i % 2:
        raise ValueError("h must have 2*I columns")
    I = two_i // 2
    dev = h.device
    if n_rows is not None:
        _dev(n_rows, "n_rows", torch.int32, numel=1, device=dev)
    T = k = 0
    if pos is not None:
        _dev(pos, "pos", torch.int32, 2, device=dev)
        T, k = pos.shape
    if row_src is not None:
        _dev(row_src, "row_src", torch.int32, numel=cap, device=dev)
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, numel=T * k, device=dev)
    if out is None:
        out = torch.empty((cap, I), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((cap, max(I // 128, 1)), dtype=torch.float32, device=dev)
    _dev(out, "out", torch.uint8, numel=cap * I, device=dev)
    _dev(scales, "scales", torch.float32, numel=cap * (I // 128), device=dev)
    _check("tk_swiglu_quant", library().tk_swiglu_quant(
        _ptr(h), cap, _ptr(n_rows), I, _ptr(row_src), _ptr(pos), _ptr(topk_w), T, k,
        _ptr(out), _ptr(scales), _stream(h)))
    return out, scales


def tk_balance_loss(logits: torch.Tensor, topk_idx: torch.Tensor, score: int,
                    f: torch.Tensor | None = None, P: torch.Tensor | None = None,
                    loss: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Per-expert load fraction f, mean normalised score P and loss = sum f*P."""
    _dev(logits, "logits", torch.float32, 2)
    T, E = logits.shape
    dev = logits.device
    _dev(topk_idx, "topk_idx", torch.int32, 2, device=dev)
    k = topk_idx.shape[1]
    if topk_idx.shape[0] != T:
        raise ValueError("topk_idx must have one row per token")
    f = torch.empty(E, dtype=torch.float32, device=dev) if f is None else f
    P = torch.empty(E, dtype=torch.float32, device=dev) if P is None else P
    loss = torch.empty(1, dtype=torch.float32, device=dev) if loss is None else loss
    need = int(library().tk_balance_workspace_bytes(T, E))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    for name, t, n in (("f", f, E), ("P", P, E), ("loss", loss, 1)):
        _dev(t, name, torch.float32, numel=n, device=dev)
    _dev(workspace, "workspace", torch.uint8, device=dev)
    _check("tk_balance_loss", library().tk_balance_loss(
        _ptr(logits), _ptr(topk_idx), T, E, k, score, _ptr(f), _ptr(P), _ptr(loss),
        _ptr(workspace), workspace.numel(), _stream(logits)))
    return f, P, loss


def _quant_shapes(rows: int, cols: int, mode: int):
    if mode in (TK_QUANT_FP8_1X128, TK_QUANT_FP8_1X128_POW2):
        return (rows, cols), torch.uint8, (rows, cols // 128)
    if mode == TK_QUANT_FP8_128X128:
        return (rows, cols), torch.uint8, ((rows + 127) // 128, cols // 128)
    if mode == TK_QUANT_FP8_PER_CHANNEL:
        return (rows, cols), torch.uint8, (cols,)
    if mode == TK_QUANT_FP4_1X32:
        return (rows, cols // 2), torch.uint8, (rows, cols // 32)
    raise ValueError(f"unknown quant mode {mode}")


def tk_quant(x: torch.Tensor, mode: int, out: torch.Tensor | None = None,
             scales: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Quantise a bf16 matrix at the granularity `mode` (TK_QUANT_*)."""
    _dev(x, "x", torch.bfloat16, 2)
    rows, cols = x.shape
    oshape, odt, sshape = _quant_shapes(rows, cols, mode)
    if out is None:
        out = torch.empty(oshape, dtype=odt, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    need = int(library().tk_quant_workspace_bytes(rows, cols, mode))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    _dev(out, "out", torch.uint8, numel=math.prod(oshape), device=x.device)
    _dev(scales, "scales", torch.float32, numel=math.prod(sshape), device=x.device)
    if workspace is not None:
        _dev(workspace, "workspace", torch.uint8, device=x.device)
    _check("tk_quant", library().tk_quant(_ptr(x), rows, cols, mode, _ptr(out), _ptr(scales),
                                          _ptr(workspace),
                                          0 if workspace is None else workspace.numel(),
                                          _stream(x)))
    return out, scales


def tk_swiglu_quant_t(h: torch.Tensor, row_src: torch.Tensor | None = None,
                      pos: torch.Tensor | None = None, topk_w: torch.Tensor | None = None,
                      out=None, scales=None, out_t=None, scales_t=None):
    """SwiGLU + 1x128 FP8 in both layouts: row-major (rows, I) and the
    transpose (I, rows) with blocks along tokens.  rows % 128 == 0."""
    _dev(h, "h", torch.bfloat16, 2)
    rows, two_i = h.shape
    I = two_i // 2
    dev = h.device
    T = k = 0
    if pos is not None:
        _dev(pos, "pos", torch.int32, 2, device=dev)
        T, k = pos.shape
    if row_src is not None:
        _dev(row_src, "row_src", torch.int32, numel=rows, device=dev)
    if topk_w is not None:
        _dev(topk_w, "topk_w", torch.float32, numel=T * k, device=dev)
    out = torch.empty((rows, I), dtype=torch.uint8, device=dev) if out is None else out
    scales = torch.empty((rows, max(I // 128, 1)), dtype=torch.float32, device=dev) if scales is None else scales
    out_t = torch.empty((I, rows), dtype=torch.uint8, device=dev) if out_t is None else out_t
    scales_t = (torch.empty((I, max(rows // 128, 1)), dtype=torch.float32, device=dev)
                if scales_t is None else scales_t)
    for name, t, dt, n in (("out", out, torch.uint8, rows * I),
                           ("scales", scales, torch.float32, rows * (I // 128)),
                           ("out_t", out_t, torch.uint8, I * rows),
                           ("scales_t", scales_t, torch.float32, I * (rows // 128))):
        _dev(t, name, dt, numel=n, device=dev)
    _check("tk_swiglu_quant_t", library().tk_swiglu_quant_t(
        _ptr(h), rows, I, _ptr(row_src), _ptr(pos), _ptr(topk_w), T, k, _ptr(out), _ptr(scales),
        _ptr(out_t), _ptr(scales_t), _stream(h)))
    return out, scales, out_t, scales_t


def tk_silu_bf16(g: torch.Tensor, out=None):
    """RN(g * sigmoid(g)) in fp32 for bf16 g (the SwiGLU kernels' sigmoid lookup)."""
    _dev(g, "g", torch.bfloat16)
    out = torch.empty(g.shape, dtype=torch.float32, device=g.device) if out is None else out
    _dev(out, "out", torch.float32, numel=g.numel(), device=g.device)
    _check("tk_silu_bf16", library().tk_silu_bf16(_ptr(g), g.numel(), _ptr(out), _stream(g)))
    return out
