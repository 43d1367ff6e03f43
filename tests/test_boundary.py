"""CPU tests of the C-ABI boundary: the library loads, exports every entry
point include/tk.h declares, and its host-side argument checks reject bad
calls before anything is launched (no GPU is touched by these calls).  Also
checks that the product package never reaches the oracle.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tk.h")
# TK_BOUNDARY_LIB: another build of the same library to check (the ASan test
# runs this file against the host-sanitised build)
LIB = os.environ.get("TK_BOUNDARY_LIB") or os.path.join(ROOT, "moe_routing_amd", "libtk.so")

ARG, UNSUP = -1, -2


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:tk_status|size_t|const char\*)\s+(tk_\w+)\s*\(",
                                 text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    L = ctypes.CDLL(LIB)
    L.tk_last_error.restype = ctypes.c_char_p
    for name in ("tk_route", "tk_map", "tk_map_aligned", "tk_expand_quant", "tk_reduce",
                 "tk_reduce_dense", "tk_expert_standin", "tk_swiglu_quant", "tk_swiglu_quant_t",
                                  "tk_silu_bf16", "tk_balance_loss",
                 "tk_quant", "tk_map_noalloc"):
        getattr(L, name).restype = ctypes.c_int32
    L.tk_map_workspace_bytes.restype = ctypes.c_size_t
    L.tk_balance_workspace_bytes.restype = ctypes.c_size_t
    L.tk_quant_workspace_bytes.restype = ctypes.c_size_t
    return L


def test_header_declares_the_entry_points():
    assert _declared() == sorted(["tk_last_error", "tk_route", "tk_map_workspace_bytes", "tk_map",
                                  "tk_map_aligned", "tk_expand_quant", "tk_reduce",
                                  "tk_reduce_dense", "tk_expert_standin", "tk_swiglu_quant", "tk_swiglu_quant_t",
                                  "tk_silu_bf16",
                                  "tk_balance_workspace_bytes", "tk_balance_loss",
                                  "tk_quant_workspace_bytes", "tk_quant", "tk_map_noalloc"])


def test_library_exports_every_declared_symbol(lib):
    for name in _declared():
        assert hasattr(lib, name), name
    # nothing but tk_* is exported (hidden visibility for the rest)
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert exported == set(_declared())


class RouteOpts(ctypes.Structure):
    _fields_ = [("score", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("group_topn", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("route_scale", ctypes.c_float)]


FAKE = ctypes.c_void_p(0x10000)        # aligned fake device address, never dereferenced
MIS = ctypes.c_void_p(0x10004)         # 4-aligned, not 16-aligned
MIS1 = ctypes.c_void_p(0x10001)


def _route(lib, T, E, k, opts, logits=FAKE, bias=None, idx=FAKE, w=FAKE):
    L = ctypes.c_int32
    return lib.tk_route(logits, bias, L(T), L(E), L(k), ctypes.byref(opts) if opts else None,
                        idx, w, None)


def test_route_rejects_bad_arguments(lib):
    o = RouteOpts(1, 8, 4, 2, 1, 2.5)
    assert _route(lib, 4, 256, 8, None) == ARG and b"opts" in lib.tk_last_error()
    assert _route(lib, -1, 256, 8, o) == ARG
    assert _route(lib, 4, 256, 0, o) == ARG
    assert _route(lib, 4, 16, 17, RouteOpts(0, 1, 1, 0, 1, 1.0)) == ARG          # k > E
    assert _route(lib, 4, 2048, 8, RouteOpts(0, 1, 1, 0, 1, 1.0)) == UNSUP       # E > max
    assert _route(lib, 4, 256, 33, RouteOpts(0, 1, 1, 0, 1, 1.0)) == UNSUP       # k > max
    assert _route(lib, 4, 250, 8, RouteOpts(1, 8, 4, 2, 1, 2.5)) == ARG          # E % groups
    assert _route(lib, 4, 256, 8, RouteOpts(1, 8, 9, 2, 1, 2.5)) == ARG          # topk_groups
    assert _route(lib, 4, 256, 8, RouteOpts(1, 8, 4, 0, 1, 2.5)) == ARG          # group_topn
    assert _route(lib, 4, 256, 40, RouteOpts(1, 8, 1, 2, 1, 2.5)) in (ARG, UNSUP)
    assert _route(lib, 4, 256, 9, RouteOpts(1, 64, 2, 2, 1, 2.5)) == ARG         # 2*4 < 9
    assert b"fewer than k" in lib.tk_last_error()
    assert _route(lib, 4, 96, 4, RouteOpts(1, 8, 4, 2, 1, 2.5)) == UNSUP         # 12/2 lanes
    assert _route(lib, 4, 256, 8, RouteOpts(7, 1, 1, 0, 1, 1.0)) == ARG          # score
    assert _route(lib, 4, 256, 8, RouteOpts(0, 1, 1, 0, 1, 1.0), bias=FAKE) == ARG
    assert _route(lib, 4, 256, 8, o, logits=None) == ARG
    assert _route(lib, 4, 256, 8, o, logits=MIS) == ARG                          # 16B for E%4==0
    assert _route(lib, 4, 256, 8, o, bias=MIS) == ARG                            # bias likewise
    assert b"16-byte" in lib.tk_last_error()
    assert _route(lib, 0, 256, 8, o, logits=None, bias=MIS, idx=None, w=None) == 0
    assert _route(lib, 4, 256, 8, o, idx=MIS1) == ARG
    assert _route(lib, 0, 256, 8, o, logits=None, idx=None, w=None) == 0         # T == 0 no-op
    assert lib.tk_last_error() == b""


def _map(lib, T, k, E, lo, hi, ws_bytes=1 << 20, counts=FAKE, ws=FAKE, idx=FAKE, pos=FAKE):
    I = ctypes.c_int32
    return lib.tk_map(idx, I(T), I(k), I(E), I(lo), I(hi), counts, FAKE, pos, None, ws,
                      ctypes.c_size_t(ws_bytes), None)


def test_last_error_is_per_thread(lib):
    # eight host threads fail tk_route with their own E at the same time (ctypes
    # drops the GIL inside the call); each must read back its own message, and
    # a successful call on a thread clears only that thread's text
    import threading
    opts = RouteOpts(1, 1, 1, 0, 1, 1.0)
    bad = []

    def worker(i):
        E = TK_MAX_EXPERTS_PLUS + i
        for n in range(500):
            if _route(lib, 4, E, 2, opts) != UNSUP or f"E={E} ".encode() not in lib.tk_last_error():
                bad.append((i, n, lib.tk_last_error()))
                return
            if n % 50 == 0:
                if _route(lib, 0, 64, 2, opts) != 0 or lib.tk_last_error() != b"":
                    bad.append((i, n, "clear", lib.tk_last_error()))
                    return

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not bad, bad[:3]


TK_MAX_EXPERTS_PLUS = 1025     # one past TK_MAX_EXPERTS


def test_map_rejects_bad_arguments(lib):
    assert _map(lib, -1, 8, 256, 0, 256) == ARG
    assert _map(lib, 4, 0, 256, 0, 256) == ARG
    assert _map(lib, 4, 33, 256, 0, 256) == UNSUP
    assert _map(lib, 4, 8, 4096, 0, 256) == UNSUP
    assert _map(lib, 4, 8, 256, 32, 32) == ARG
    assert _map(lib, 4, 8, 256, -1, 32) == ARG
    assert _map(lib, 4, 8, 256, 0, 257) == ARG
    assert _map(lib, 8192, 8, 256, 0, 256, ws_bytes=100) == ARG
    assert b"workspace" in lib.tk_last_error()
    assert _map(lib, 4, 8, 256, 0, 256, counts=None) == ARG
    assert _map(lib, 4, 8, 256, 0, 256, ws=MIS1) == ARG
    assert _map(lib, 4, 8, 256, 0, 256, ws=MIS) == ARG     # workspace needs 16-byte alignment
    assert _map(lib, 4, 8, 256, 0, 256, idx=None) == ARG


def test_map_noalloc_rejects_bad_arguments_and_sizes(lib):
    # the argument checks of tk_map, then the size of the library's scratch
    # array, all before any device call (these run without a GPU)
    I = ctypes.c_int32

    def call(T, k, E, lo, hi, counts=FAKE, idx=FAKE, pos=FAKE):
        return lib.tk_map_noalloc(idx, I(T), I(k), I(E), I(lo), I(hi), counts, FAKE, pos, None,
                                  None)
    assert call(-1, 8, 256, 0, 256) == ARG
    assert call(4, 0, 256, 0, 256) == ARG
    assert call(4, 33, 256, 0, 256) == UNSUP
    assert call(4, 8, 256, 32, 32) == ARG
    assert call(4, 8, 256, 0, 256, counts=None) == ARG
    assert call(4, 8, 256, 0, 256, idx=MIS1) == ARG
    # 1 MiB holds the count matrix up to T*n_local/256 + n_local ints = 2^18
    assert lib.tk_map_workspace_bytes(261120, 8, 256) <= 1 << 20
    assert call(262144, 8, 256, 0, 256) == ARG
    assert b"scratch" in lib.tk_last_error()
    assert call(200000, 8, 1024, 0, 1024) == ARG


def test_map_workspace_bytes(lib):
    # per-tile counts, one row of n_local ints per tile, plus one int per
    # local expert
    f = lib.tk_map_workspace_bytes
    assert f(0, 8, 256) == 0
    assert f(8192, 8, 256) == (32 * 256 + 256) * 4     # 32 tiles of 256 tokens
    assert f(32768, 8, 32) == (128 * 32 + 32) * 4      # 128 tiles of 256 tokens
    assert f(1, 1, 1024) == (1 * 1024 + 1024) * 4      # one tile
    # the largest T the int32 positions allow (k = 1): tile counts in 64 bits
    big = 2**31 - 1
    assert f(big, 1, 256) == ((big + 255) // 256 * 256 + 256) * 4
    assert lib.tk_balance_workspace_bytes(big, 256) > 0


def _expand(lib, T, H, k, mode, cap, x=FAKE, out=FAKE, scales=FAKE, pos=FAKE):
    I = ctypes.c_int32
    return lib.tk_expand_quant(x, I(T), I(H), I(k), pos, I(mode), out, scales,
                               ctypes.c_int64(cap), None)


def test_expand_rejects_bad_arguments(lib):
    assert _expand(lib, -1, 256, 2, 0, 8) == ARG
    assert _expand(lib, 4, 200, 2, 1, 8) == ARG                       # H % 128 in FP8
    assert b"128" in lib.tk_last_error()
    assert _expand(lib, 4, 260, 2, 0, 8) == ARG                       # H % 8
    assert _expand(lib, 4, 256, 2, 5, 8) == ARG                       # mode
    assert _expand(lib, 4, 256, 2, 1, 8, scales=None) == ARG
    assert _expand(lib, 4, 256, 2, 1, -1) == ARG
    assert _expand(lib, 4, 256, 2, 1, 8, out=MIS) == ARG
    assert _expand(lib, 4, 256, 2, 1, 8, x=None) == ARG
    assert _expand(lib, 4, 256, 40, 1, 8) == UNSUP
    assert _expand(lib, 0, 256, 2, 1, 8, x=None, out=None, pos=None) == 0


@pytest.mark.parametrize("fn", ["tk_reduce", "tk_reduce_dense"])
def test_reduce_and_standin_reject_bad_arguments(lib, fn):
    I = ctypes.c_int32
    r = lambda T, k, H, rows=8, y=FAKE, out=FAKE: getattr(lib, fn)(
        y, ctypes.c_int64(rows), FAKE, FAKE, I(T), I(k), I(H), out, None)
    assert r(-1, 2, 256) == ARG
    assert r(4, 0, 256) == ARG
    assert r(4, 33, 256) == UNSUP
    assert r(4, 2, 12) == ARG
    assert r(4, 2, 256, rows=-1) == ARG
    assert r(4, 2, 256, out=MIS) == ARG
    assert r(4, 2, 256, y=None) == ARG
    assert r(0, 2, 256, y=None, out=None) == 0
    s = lambda cap, H, xq=FAKE: lib.tk_expert_standin(xq, FAKE, FAKE, ctypes.c_int64(cap), I(H),
                                                      ctypes.c_float(0.5), FAKE, None)
    assert s(8, 100) == ARG
    assert s(-1, 128) == ARG
    assert s(8, 128, xq=None) == ARG
    assert s(8, 128, xq=MIS) == ARG
    assert s(0, 128) == 0


def test_product_path_never_uses_the_oracle():
    pkg = os.path.join(ROOT, "moe_routing_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"import\s+oracle|from\s+oracle|liboracle|\borc_\w+",
                                     text), f


def _swiglu(lib, cap, I, h=FAKE, n_rows=None, row_src=None, pos=None, w=None, T=0, k=0, out=FAKE,
            scales=FAKE):
    I32 = ctypes.c_int32
    return lib.tk_swiglu_quant(h, ctypes.c_int64(cap), n_rows, I32(I), row_src, pos, w, I32(T),
                               I32(k), out, scales, None)


def test_swiglu_rejects_bad_arguments(lib):
    assert _swiglu(lib, -1, 256) == ARG
    assert _swiglu(lib, 8, 0) == ARG
    assert _swiglu(lib, 8, 200) == ARG                       # I % 128 != 0
    assert _swiglu(lib, 8, 256, row_src=FAKE) == ARG         # weights need all three
    assert b"together" in lib.tk_last_error()
    assert _swiglu(lib, 8, 256, row_src=FAKE, pos=FAKE, w=FAKE, T=4, k=0) == ARG
    assert _swiglu(lib, 8, 256, row_src=FAKE, pos=FAKE, w=FAKE, T=4, k=33) == ARG
    assert _swiglu(lib, 8, 256, h=None) == ARG
    assert _swiglu(lib, 8, 256, out=MIS) == ARG
    assert _swiglu(lib, 8, 256, scales=MIS1) == ARG
    assert _swiglu(lib, 0, 256, h=None, out=None, scales=None) == 0   # nothing to do


def test_map_aligned_rejects_bad_arguments(lib):
    I = ctypes.c_int32
    ws = ctypes.c_size_t(1 << 20)

    def call(T, k, E, lo, hi, align):
        return lib.tk_map_aligned(FAKE, I(T), I(k), I(E), I(lo), I(hi), I(align), FAKE, FAKE,
                                  FAKE, None, FAKE, ws, None)

    assert call(4, 8, 256, 0, 256, 0) == ARG
    assert call(4, 8, 256, 0, 256, -3) == ARG
    # T*k plus the largest padding must fit in int32 positions
    assert call(1 << 27, 8, 256, 0, 256, 1 << 24) == ARG
    assert b"padding" in lib.tk_last_error()


def test_balance_rejects_bad_arguments(lib):
    I = ctypes.c_int32
    ws = ctypes.c_size_t(1 << 20)

    def call(T, E, k, score, logits=FAKE, idx=FAKE, w=FAKE, wsb=ws):
        return lib.tk_balance_loss(logits, idx, I(T), I(E), I(k), I(score), FAKE, FAKE, FAKE, w,
                                   wsb, None)

    assert call(0, 256, 8, 1) == ARG
    assert call(16, 0, 8, 1) == ARG
    assert call(16, 2048, 8, 1) == UNSUP
    assert call(16, 256, 0, 1) == ARG
    assert call(16, 256, 8, 7) == ARG
    assert call(16, 256, 8, 1, logits=None) == ARG
    assert call(8192, 256, 8, 1, wsb=ctypes.c_size_t(10)) == ARG
    assert b"workspace" in lib.tk_last_error()
    assert call(16, 256, 8, 1, w=MIS1) == ARG
    assert lib.tk_balance_workspace_bytes(I(8192), I(256)) == 256 * 256 * 8 + 16   # 256 tiles of 32 + counter
    assert lib.tk_balance_workspace_bytes(I(0), I(256)) == 0


def test_quant_rejects_bad_arguments(lib):
    I, I64 = ctypes.c_int32, ctypes.c_int64

    def call(rows, cols, mode, x=FAKE, out=FAKE, sc=FAKE, ws=None, wsb=0):
        return lib.tk_quant(x, I64(rows), I(cols), I(mode), out, sc, ws, ctypes.c_size_t(wsb), None)

    assert call(-1, 256, 0) == ARG
    assert call(4, 256, 9) == ARG
    assert call(4, 200, 0) == ARG                 # FP8 blocks need cols % 128 == 0
    assert call(4, 48, 4) == ARG                  # FP4 blocks need cols % 32 == 0
    assert call(4, 12, 3) == ARG                  # per-channel needs cols % 8 == 0
    assert call(4, 256, 0, x=None) == ARG
    assert call(4, 256, 0, out=MIS) == ARG
    assert call(4, 256, 3) == ARG                 # per-channel without workspace
    assert b"workspace" in lib.tk_last_error()
    assert call(0, 256, 0, x=None, out=None, sc=None) == 0
    f = lib.tk_quant_workspace_bytes
    assert f(I64(1000), I(256), I(3)) == 9 * 256 * 4      # 8 chunks of 128 rows + reciprocals
    assert f(I64(1000), I(256), I(0)) == 0


def test_swiglu_t_rejects_bad_arguments(lib):
    I32, I64 = ctypes.c_int32, ctypes.c_int64

    def call(rows, I, rs=None, pos=None, w=None, T=0, k=0, h=FAKE, out=FAKE, out_t=FAKE):
        return lib.tk_swiglu_quant_t(h, I64(rows), I32(I), rs, pos, w, I32(T), I32(k), out, FAKE,
                                     out_t, FAKE, None)

    assert call(100, 256) == ARG                  # rows % 128 != 0
    assert call(-128, 256) == ARG
    assert call(128, 200) == ARG
    assert call(128, 256, rs=FAKE) == ARG
    assert call(128, 256, h=None) == ARG
    assert call(128, 256, out_t=MIS) == ARG
    assert call(0, 256, h=None, out=None, out_t=None) == 0


def test_silu_rejects_bad_arguments(lib):
    f = lib.tk_silu_bf16
    I64 = ctypes.c_int64
    assert f(FAKE, I64(-1), FAKE, None) == ARG
    assert f(None, I64(4), FAKE, None) == ARG
    assert f(FAKE, I64(4), None, None) == ARG
    assert f(FAKE, I64(4), MIS1, None) == ARG         # out not 4-byte aligned
    assert f(MIS1, I64(4), FAKE, None) == ARG         # g not 2-byte aligned
    assert f(None, I64(0), None, None) == 0


def test_calibration_library_exports_only_the_stream_copy():
    """bench.py's reference copy lives in its own library, outside the routing ABI."""
    import subprocess
    from moe_routing_amd import _build
    if not os.path.exists(_build.CALIB_LIB):
        pytest.skip("library not built")
    out = subprocess.run(["nm", "-D", "--defined-only", _build.CALIB_LIB], capture_output=True,
                         text=True).stdout
    assert {l.split()[-1] for l in out.splitlines() if " T " in l} == {"tk_calib_stream_copy"}
    lib = ctypes.CDLL(_build.CALIB_LIB)
    f = lib.tk_calib_stream_copy
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert f(None, None, 0, None) == 0                       # nothing to copy
    assert f(FAKE, FAKE, 24, None) == -1                     # not a multiple of 16
    assert f(MIS, FAKE, 32, None) == -1                      # misaligned source
    assert f(None, FAKE, 32, None) == -1


def test_bench_refuses_more_than_one_gpu():
    # one GPU's path: --gpus N > 1 ends with a message and status 2, before
    # anything touches a device
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_c_program_uses_the_header_and_library(lib, tmp_path):
    # include/tk.h is a C header: a C11 program built with -pedantic -Werror
    # (the ROCm headers taken as system headers) links libtk.so and sees the
    # same status codes, per-thread messages, size queries and tk_route_opts
    # layout as the ctypes binding
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    lib_dir = os.path.join(ROOT, "moe_routing_amd")
    exe = str(tmp_path / "abi_consumer")
    subprocess.run([gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-isystem", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "helpers", "abi_consumer.c"), "-o", exe,
                    "-L", lib_dir, "-ltk", f"-Wl,-rpath,{lib_dir}"], check=True, timeout=120)
    out = subprocess.run([exe], capture_output=True, text=True, check=True, timeout=60).stdout
    got = {}
    for line in out.splitlines():
        name, *vals = line.split()
        got[name] = [int(v) for v in vals]
    assert got["initial_error_empty"] == [1]
    assert got["opts_size"] == [ctypes.sizeof(RouteOpts)]
    assert got["opts_scale_offset"] == [RouteOpts.route_scale.offset]
    assert got["route_null_opts"] == [ARG, 1]
    assert got["route_too_many_experts"] == [UNSUP, 1]
    assert got["reduce_bad_h"] == [ARG, 1]
    assert got["reduce_no_tokens"] == [0, 0]          # a no-op, and the message cleared
    assert got["expand_bad_mode"] == [ARG, 1]
    L = ctypes.c_int32
    assert got["map_ws"] == [lib.tk_map_workspace_bytes(L(8192), L(8), L(256))]
    assert got["balance_ws"] == [lib.tk_balance_workspace_bytes(L(8192), L(256))]
    lib.tk_quant_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32]
    pc = int(re.search(r"#define TK_QUANT_FP8_PER_CHANNEL (\d+)", open(HEADER).read()).group(1))
    assert got["quant_pc_ws"] == [lib.tk_quant_workspace_bytes(8192, 7168, pc)]


def test_recorded_combine_traffic_matches_its_code():
    # bench.py reports the combine's measured HBM traffic only while the
    # committed counter summary was taken on the combine's current code
    import sys
    sys.path.insert(0, ROOT)
    import bench
    assert bench.measured_traffic() is not None, (
        "profiles/hbm_counters_v3_T8192.md was taken on other combine code: re-collect it")
