#!/usr/bin/env python3
"""Benchmark of the MoE routing hot path on one MI355X.

One step = the whole path over one batch of the DeepSeek-V3-shaped workload
(T=8192 tokens, hidden H=7168, E=256 experts in 8 groups of 32, top-8):

  tk_route         sigmoid scores + per-expert bias, top-2 group sums, top-4
                   groups, top-8 experts, weights normalised * 2.5
  tk_map           counts, offsets, stable positions (no mask: all local)
  tk_expand_quant  1x128 FP8 E4M3 expand into 65536 expert-contiguous rows
  tk_reduce_dense  bf16 combine of 65536 expert-output rows, fp32 accumulate
                   (tk_reduce's dense form: every slot has a row here; two
                   launches of 4096 tokens on 256 compute units)

Inputs are synthetic (seeded normal logits, U(-0.1,0.1) bias, bf16 N(0,1)
hidden states with 1 % outlier rows x50, bf16 N(0,1) expert outputs) and
resident in HBM before the timed region.  The expert GEMMs are not part of
the path: the reduce consumes a fixed expert-output tensor.

Prints ONE JSON line: routed tokens/s (value: passes that each start with
the MALL and L2 evicted, one pair of HIP events around each), the pipeline's
algorithmic HBM GB/s, the same passes back to back (warm: x then stays in the
MALL), per-kernel times from HIP events recorded between the calls (mean,
median, p10, p90; warm and cold), the rate of the repository's streaming copy
kernel for reference (stream_copy), the roofline of the dominant kernel (the
reduce, per launch), the CPU oracle's rate (one thread, and all host cores on token
shards) and the comparison of the step's GPU outputs with the oracle's
outputs for the same inputs (parity; a mismatch makes the exit status 1).
Steps beyond the routing path (next_rows) are timed separately on the same data and do not
enter value: SwiGLU + 1x128 FP8 quantisation of the 65536 expanded rows at
the DeepSeek-V3 expert width I = 2048 (plain and transposing), weighted by the
routing weights through the step's map; the padded map; the balance loss;
the other quantisation granularities of the hidden states; the expand without
quantisation (bf16 rows); both combines (tk_reduce_dense, the step's, and
tk_reduce) on the step's data; one GPU's share of an expert-parallel step
(T = 32768, experts 32..63 local, with the stand-in expert); and the step at
decode-like batch sizes (the first 64 and 256 tokens).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

T, H, E, K = 8192, 7168, 256, 8
R = T * K
NB = H // 128
PEAK_HBM_GBPS = 8000.0

# Algorithmic bytes per launch (each token read once, each expanded row written
# once, each expert-output row read once; workspace traffic excluded).
BYTES = {
    "route": T * E * 4 + E * 4 + T * K * (4 + 4),
    "map": T * K * 4 + T * K * 4 + R * 4 + (2 * E + 1) * 4,
    "expand": T * H * 2 + R * H + R * NB * 4 + T * K * 4,
    "reduce": R * H * 2 + T * K * 8 + T * H * 2,
}
BYTES["total"] = sum(BYTES.values())
WORKLOAD = (f"DeepSeek-V3 MoE routing hot path: T={T} H={H} E={E} (8 groups x 32) k={K}; "
            "sigmoid+bias gating, top-4 groups, weights x2.5; stable map; "
            "1x128 FP8 E4M3 expand; bf16 combine with fp32 accumulation")

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_counters_v3_T8192.md")


def kernel_source_hash() -> str:
    """Hash of the combine's code (reduce.hip, tk_internal.h) with comments and
    whitespace removed, so that an edit of comments alone keeps the counters."""
    h = hashlib.sha256()
    for f in ("reduce.hip", "tk_internal.h"):
        with open(os.path.join(ROOT, "moe_routing_amd", "csrc", f)) as fh:
            code = re.sub(r"/\*.*?\*/", " ", fh.read(), flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per reduce launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's
    reading), or None when absent or taken on different reduce sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    kv = {}
    for line in lines:
        if ":" in line and not line.startswith(("#", "|", "`")):
            key, _, val = line.partition(":")
            kv[key.strip()] = val.strip()
    if kv.get("reduce_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(kv["reduce_hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _progress(msg: str) -> None:
    """A progress line on stderr (the JSON line alone goes to stdout)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def cpu_baseline(inputs, reps: int = 2):
    """The oracle, as it stands, on full steps of the workload: one thread,
    then all host cores (at most 16).  The all-cores leg calls the same oracle
    functions on token shards from a thread pool -- route, expand and reduce
    are independent per token, and ctypes releases the interpreter lock
    around each C call -- with the map run serially; its outputs are checked
    equal to the one-thread run's.  Returns the report and the one-thread
    run's outputs, against which the GPU step's outputs are then compared."""
    import ctypes
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    import oracle
    logits, bias, x, y, r = inputs
    t_rm = t_ex = t_rd = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        idx, w = oracle.route(logits, bias, K, **r)
        counts, offsets, pos, row_src = oracle.map_routes(idx, E)
        t1 = time.perf_counter()
        xq, sc = oracle.expand(x, pos, 1, R)
        t2 = time.perf_counter()
        out = oracle.reduce(y, pos, w.astype(np.float32))
        t3 = time.perf_counter()
        t_rm += t1 - t0
        t_ex += t2 - t1
        t_rd += t3 - t2
    secs = (t_rm + t_ex + t_rd) / reps
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), model)
    except OSError:
        pass

    n = max(1, min(16, os.cpu_count() or 1))
    shards = [(T * i // n, T * (i + 1) // n) for i in range(n)]
    L = oracle.lib()
    xs = np.ascontiguousarray(x)
    xq_m = np.zeros((R, H), np.uint8)
    sc_m = np.zeros((R, NB), np.float32)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    m_rm = m_ex = m_rd = 0.0
    with ThreadPoolExecutor(n) as ex:
        for _ in range(reps):
            t0 = time.perf_counter()
            parts = list(ex.map(lambda s: oracle.route(logits[s[0]:s[1]], bias, K, **r), shards))
            idx_m = np.concatenate([p[0] for p in parts])
            w_m = np.concatenate([p[1] for p in parts])
            _, _, pos_m, _ = oracle.map_routes(idx_m, E)
            t1 = time.perf_counter()

            def expand_shard(s):
                rc = L.orc_expand(ptr(xs[s[0]:]), s[1] - s[0], H, K, ptr(pos_m[s[0]:]), 1, R,
                                  ptr(xq_m), ptr(sc_m))
                assert rc == 0
            list(ex.map(expand_shard, shards))
            t2 = time.perf_counter()
            w32 = w_m.astype(np.float32)
            out_m = np.concatenate(list(ex.map(
                lambda s: oracle.reduce(y, pos_m[s[0]:s[1]], w32[s[0]:s[1]]), shards)))
            t3 = time.perf_counter()
            m_rm += t1 - t0
            m_ex += t2 - t1
            m_rd += t3 - t2
    same = bool(np.array_equal(idx_m, idx) and np.array_equal(w_m, w) and np.array_equal(pos_m, pos)
                and np.array_equal(xq_m, xq) and np.array_equal(sc_m, sc) and np.array_equal(out_m, out))
    del xq_m, sc_m, out_m
    m_secs = (m_rm + m_ex + m_rd) / reps
    report = {"value": round(T / secs, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
              "host": f"{model}, {os.cpu_count()} logical CPUs visible",
              "sample": f"{reps} full steps (T={T} each) of route+map+expand(FP8)+reduce through the "
                        f"single-threaded C oracle, mean per step: route+map {t_rm / reps:.2f}s, "
                        f"expand {t_ex / reps:.2f}s, reduce {t_rd / reps:.2f}s",
              "all_cores": {"value": round(T / m_secs, 1), "unit": "tokens/s", "cores": n,
                            "kind": "oracle", "identical_to_one_thread": same,
                            "sample": f"the same {reps} steps, the oracle's route, expand and reduce "
                                      f"on {n} token shards in {n} threads, map serial; mean per "
                                      f"step: route+map {m_rm / reps:.2f}s, expand {m_ex / reps:.2f}s, "
                                      f"reduce {m_rd / reps:.2f}s"}}
    outs = {"idx": idx, "w": w, "counts": counts, "offsets": offsets, "pos": pos,
            "row_src": row_src, "xq": xq, "sc": sc, "out": out}
    return report, outs


# Parity bars of the step against the oracle: integer and byte outputs
# bit-exact; weights (fp32 against the oracle's fp64) within W_RTOL; the
# combine per element within COMBINE_ATOL + COMBINE_RTOL * |ref| in bf16.
W_RTOL, W_ATOL = 4e-6, 1e-9
COMBINE_ATOL = COMBINE_RTOL = 1e-2


def _bf16_bits_to_f64(h):
    import numpy as np
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def step_parity(gpu: dict, ref: dict) -> dict:
    """Compare the timed step's GPU outputs with the oracle's outputs for the
    same inputs (numpy comparisons only)."""
    import numpy as np
    exact = {n: bool(np.array_equal(gpu[n], ref[n]))
             for n in ("idx", "counts", "offsets", "pos", "row_src", "xq", "sc")}
    w_ok = bool(np.allclose(gpu["w"], ref["w"], rtol=W_RTOL, atol=W_ATOL))
    w_rel = float(np.max(np.abs(gpu["w"].astype(np.float64) - ref["w"]) /
                         np.maximum(np.abs(ref["w"]), 1e-30)))
    g = _bf16_bits_to_f64(gpu["out"])
    r = _bf16_bits_to_f64(ref["out"])
    err = np.abs(g - r)
    ok = err <= COMBINE_ATOL + COMBINE_RTOL * np.abs(r)
    combine = {"tokens": int(gpu["out"].shape[0]), "allclose": bool(ok.all()),
               "n_outside": int((~ok).sum()),
               "max_abs": float(err.max(initial=0.0)),
               "max_rel": float((err / np.maximum(np.abs(r), 1e-30)).max(initial=0.0)),
               "bit_exact_frac": float((gpu["out"] == ref["out"]).mean())}
    return {"ok": all(exact.values()) and w_ok and combine["allclose"],
            "bit_exact": exact, "weights_within_rtol": w_ok, "weights_max_rel": w_rel,
            "combine": combine,
            "bars": f"idx, counts, offsets, pos, row_src, FP8 codes and scales bit-exact; weights "
                    f"rtol {W_RTOL}; combine |gpu-ref| <= {COMBINE_ATOL} + {COMBINE_RTOL}*|ref| "
                    f"on every element of the ({T}, {H}) output"}


SWIGLU_I = 2048   # DeepSeek-V3's expert width


def bench_swiglu(tk, torch, y, n_rows, row_src, pos, w, steps):
    """SwiGLU + 1x128 FP8 over the step's expanded rows (weighted), plain and
    transposing forms.  The sigmoid is a table lookup, so both stream: each
    is priced against HBM with its algorithmic bytes (h read once, codes and
    scales written once, the routing metadata read once)."""
    I = SWIGLU_I
    h = y.view(-1)[: R * 2 * I].view(R, 2 * I)      # N(0,1) bf16 rows of width 2*I
    q = torch.empty((R, I), dtype=torch.uint8, device=y.device)
    s = torch.empty((R, I // 128), dtype=torch.float32, device=y.device)
    n = min(steps, 20)
    us = _time_calls(torch, lambda: tk.tk_swiglu_quant(h, n_rows, row_src, pos, w, q, s), n, (q, s))
    nbytes = R * 2 * I * 2 + R * I + R * (I // 128) * 4 + R * 4 + T * K * 8

    def roof(kernel, nb, t):
        return {"kernel": kernel, "bound": "hbm", "achieved": round(nb / t / 1e3, 1),
                "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(nb / t / 1e3 / PEAK_HBM_GBPS, 4)}

    # the transposing form: both layouts from one read of h
    qt = torch.empty((I, R), dtype=torch.uint8, device=y.device)
    st = torch.empty((I, R // 128), dtype=torch.float32, device=y.device)
    us_t = _time_calls(torch, lambda: tk.tk_swiglu_quant_t(h, row_src, pos, w, q, s, qt, st),
                       n, (q, s, qt, st))
    nbytes_t = nbytes + R * I + I * (R // 128) * 4
    transposed = {"workload": f"as above, plus a^T ({I}, {R}) in 1x128 blocks along tokens",
                  "us_per_call": round(us_t, 2), "timing": "HIP graph of the calls",
                  "algorithmic_bytes": nbytes_t,
                  "roofline": roof("swiglu_quant_t_kernel<true>", nbytes_t, us_t)}
    return {"workload": f"{R} expanded rows of the step's routing, I={I} (gate|up bf16 -> "
                        "E4M3 + fp32 1x128 scales), routing weights applied",
            "us_per_call": round(us, 2), "timing": "HIP graph of the calls",
            "algorithmic_bytes": nbytes,
            "roofline": roof("swiglu_quant_kernel<true>", nbytes, us),
            "transposed": transposed}


def stream_copy_gbps(torch, dev, reps: int = 10):
    """Bandwidth of the repository's streaming copy kernel over 1 GiB: read +
    written bytes per second (the reference for what a plain copy reaches)."""
    import ctypes
    from moe_routing_amd import _build
    if not os.path.exists(_build.CALIB_LIB):
        return None
    lib = ctypes.CDLL(_build.CALIB_LIB)
    lib.tk_calib_stream_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                         ctypes.c_void_p]
    lib.tk_calib_stream_copy.restype = ctypes.c_int
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream

    def copy():
        if lib.tk_calib_stream_copy(src.data_ptr(), dst.data_ptr(), n, stream) != 0:
            raise RuntimeError("stream copy failed")

    copy()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        copy()
    b.record()
    torch.cuda.synchronize()
    if not torch.equal(src[:4096], dst[:4096]) or not torch.equal(src[-4096:], dst[-4096:]):
        raise RuntimeError("stream copy wrote wrong bytes")
    return 2.0 * n * reps / (a.elapsed_time(b) * 1e-3) / 1e9


def _time_calls(torch, call, steps, outputs):
    """GPU time per call of a short, launch-bound call: `steps` calls are
    captured in one HIP graph and the graph is replayed, so the host-side cost
    of the Python binding does not leave the GPU idle between calls.  The
    graph's outputs are checked against an eager call first."""
    call()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up on a side stream before capture
        for _ in range(2):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(steps):
            call()
    g.replay()
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(eager, outputs)):
        raise RuntimeError("graph replay differs from the eager call")
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / steps


def bench_map_balance(tk, torch, logits, idx, steps):
    """The map with expert segments padded to 128 rows (grouped-GEMM layout),
    and the load-balance statistics + loss, on the step's routing."""
    dev = logits.device
    align = 128
    cap = T * K + E * (align - 1)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T, K), dtype=torch.int32, device=dev)
    row_src = torch.empty(cap, dtype=torch.int32, device=dev)
    ws = torch.empty(max(tk.tk_map_workspace_bytes(T, K, E), 16), dtype=torch.uint8, device=dev)
    us_map = _time_calls(torch, lambda: tk.tk_map_aligned(idx, E, 0, E, align, counts, offsets,
                                                          pos, row_src, ws), steps,
                         (counts, offsets, pos))
    f = torch.empty(E, dtype=torch.float32, device=dev)
    P = torch.empty(E, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    wsb = torch.empty(max(tk.library().tk_balance_workspace_bytes(T, E), 16), dtype=torch.uint8,
                      device=dev)
    us_bal = _time_calls(torch, lambda: tk.tk_balance_loss(logits, idx, tk.TK_SCORE_SIGMOID, f, P,
                                                           loss, wsb), steps, (f, P, loss))
    bal_bytes = T * E * 4 + T * K * 4 + 2 * E * 4 + 4
    return {"map_aligned_128": {"workload": f"T={T}, k={K}, E={E}, segments padded to {align} rows",
                                "us_per_call": round(us_map, 2), "timing": "HIP graph of the calls",
                                "bound": "latency (two dependent launches)"},
            "balance_loss": {"workload": f"T={T}, E={E}, k={K}, sigmoid scores",
                             "us_per_call": round(us_bal, 2), "timing": "HIP graph of the calls",
                             "hbm_gbps": round(bal_bytes / us_bal / 1e3, 1),
                             "bound": "latency (two dependent launches)"}}


def bench_expand_bf16(tk, torch, x, pos, steps):
    """The expand without quantisation (bf16 rows), on the step's routing."""
    out = torch.empty((R, H), dtype=torch.bfloat16, device=x.device)
    us = _time_calls(torch, lambda: tk.tk_expand_quant(x, pos, tk.TK_EXPAND_BF16, R, out),
                     min(steps, 20), (out,))
    nbytes = T * H * 2 + R * H * 2 + T * K * 4
    del out
    return {"expand_bf16": {"workload": f"x bf16 ({T}, {H}) -> {R} bf16 rows, the step's routing",
                            "us_per_call": round(us, 2), "timing": "HIP graph of the calls",
                            "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1),
                                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                         "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                                         "algorithmic_bytes": nbytes}}}


def bench_combines(tk, torch, y, pos, w, steps):
    """Both combines on the step's data, each as a HIP graph of the calls:
    tk_reduce_dense (the step's) and tk_reduce (one wave per unit, the form
    for routings where most slots are masked)."""
    res = {}
    for name in ("tk_reduce_dense", "tk_reduce"):
        out = torch.empty((T, H), dtype=torch.bfloat16, device=y.device)
        fn = getattr(tk, name)
        us = _time_calls(torch, lambda: fn(y, pos, w, out), min(steps, 20), (out,))
        nb = BYTES["reduce"]
        res[name] = {"us_per_call": round(us, 2), "hbm_gbps": round(nb / us / 1e3, 1),
                     "frac": round(nb / us / 1e3 / PEAK_HBM_GBPS, 4)}
    return {"combines": {"workload": f"the step's combine: y bf16 ({R}, {H}), k={K}, T={T}",
                         "timing": "HIP graph of the calls", **res}}


def bench_ep_share(tk, torch, np, synth, dev, steps):
    """The one-GPU share of an expert-parallel step: DeepSeek-V3 routing over
    T = 32768 tokens with experts 32..63 local (a log-Zipf popularity offset on
    the logits), the map with the local mask, the FP8 expand of the local
    routes, the stand-in expert (dequantise x 0.5) and the combine of the local
    routes.  The time includes the stand-in; the bytes leave it out and count x
    only for the tokens with at least one local route."""
    cfg = synth.ep_share(0)
    T4, E4, K4, H4 = cfg["T"], cfg["E"], cfg["k"], cfg["H"]
    lo, hi = cfg["local"]
    nl = hi - lo
    logits = torch.from_numpy(cfg["logits"]).to(dev)
    x = torch.from_numpy(cfg["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    del cfg["x"]
    opts = tk.RouteOpts(**cfg["route"])
    cap = T4 * K4                               # every route local, at worst
    idx = torch.empty((T4, K4), dtype=torch.int32, device=dev)
    w = torch.empty((T4, K4), dtype=torch.float32, device=dev)
    counts = torch.empty(nl, dtype=torch.int32, device=dev)
    offsets = torch.empty(nl + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T4, K4), dtype=torch.int32, device=dev)
    row_src = torch.empty(cap, dtype=torch.int32, device=dev)
    ws = torch.empty(max(tk.tk_map_workspace_bytes(T4, K4, nl), 16), dtype=torch.uint8, device=dev)
    xq = torch.empty((cap, H4), dtype=torch.uint8, device=dev)
    sc = torch.empty((cap, H4 // 128), dtype=torch.float32, device=dev)
    y = torch.empty((cap, H4), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T4, H4), dtype=torch.bfloat16, device=dev)

    names = ("route", "map", "expand", "standin", "reduce")

    def step(ev=None):
        calls = (lambda: tk.tk_route(logits, None, K4, opts, idx, w),
                 lambda: tk.tk_map(idx, E4, lo, hi, counts, offsets, pos, row_src, ws),
                 lambda: tk.tk_expand_quant(x, pos, tk.TK_EXPAND_FP8_E4M3_1X128, cap, xq, sc),
                 lambda: tk.tk_expert_standin(xq, sc, offsets[nl:], 0.5, y),
                 lambda: tk.tk_reduce(y, pos, w, out))
        for i, c in enumerate(calls):
            if ev is not None:
                ev[i].record()
            c()
        if ev is not None:
            ev[len(calls)].record()

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    n = min(steps, 20)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        step()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / n
    per = {m: [] for m in names}
    for _ in range(n):                          # breakdown: an event between calls
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
        step(ev)
        torch.cuda.synchronize()
        for i, m in enumerate(names):
            per[m].append(ev[i].elapsed_time(ev[i + 1]) * 1e3)
    kern = {m: round(float(np.median(v)), 2) for m, v in per.items()}
    r_loc = int(offsets[nl].item())
    t_act = int((pos >= 0).any(dim=1).sum().item())
    nbytes = (T4 * E4 * 4 + T4 * K4 * 8                                   # route
              + T4 * K4 * 8 + r_loc * 4 + (2 * nl + 1) * 4                # map
              + t_act * H4 * 2 + r_loc * H4 + r_loc * (H4 // 128) * 4 + T4 * K4 * 4   # expand
              + r_loc * H4 * 2 + T4 * K4 * 8 + T4 * H4 * 2)               # reduce
    return {"ep_share_T32768": {
        "workload": f"T={T4} H={H4} E={E4} k={K4}, experts [{lo}, {hi}) local; route, masked map, "
                    "FP8 expand, stand-in expert, combine",
        "us_per_step": round(us, 2), "timing": "back-to-back steps between two events",
        "rows_local": r_loc, "tokens_with_local_routes": t_act,
        "algorithmic_bytes_without_standin": nbytes,
        "hbm_gbps": round(nbytes / us / 1e3, 1),
        "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4),
        "kernel_us_median": kern,
        "hbm_frac_without_standin_time": round(
            nbytes / (us - kern["standin"]) / 1e3 / PEAK_HBM_GBPS, 4)}}


def bench_small_batch(tk, torch, logits, bias, x, y, opts, steps):
    """The routing step at decode-like batch sizes: the first Ts tokens of the
    same workload (Ts = 64 and 256, one map tile, so the map is one launch),
    route + map + FP8 expand + combine, timed per step as a HIP graph (the
    step is launch-bound; eager Python launches would dominate)."""
    dev = logits.device
    res = {}
    for Ts in (64, 256):
        R_s = Ts * K
        idx = torch.empty((Ts, K), dtype=torch.int32, device=dev)
        w = torch.empty((Ts, K), dtype=torch.float32, device=dev)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        pos = torch.empty((Ts, K), dtype=torch.int32, device=dev)
        row_src = torch.empty(R_s, dtype=torch.int32, device=dev)
        ws = torch.empty(max(tk.tk_map_workspace_bytes(Ts, K, E), 16), dtype=torch.uint8,
                         device=dev)
        xq = torch.empty((R_s, H), dtype=torch.uint8, device=dev)
        sc = torch.empty((R_s, NB), dtype=torch.float32, device=dev)
        out = torch.empty((Ts, H), dtype=torch.bfloat16, device=dev)
        lg, xs, ys = logits[:Ts], x[:Ts], y[:R_s]

        def call():
            tk.tk_route(lg, bias, K, opts, idx, w)
            tk.tk_map(idx, E, 0, E, counts, offsets, pos, row_src, ws)
            tk.tk_expand_quant(xs, pos, tk.TK_EXPAND_FP8_E4M3_1X128, R_s, xq, sc)
            tk.tk_reduce(ys, pos, w, out)

        us = _time_calls(torch, call, steps, [idx, w, pos, row_src, xq, sc, out])
        res[f"T{Ts}"] = {"us_per_step": round(us, 2), "tokens_per_s": round(Ts / us * 1e6, 1)}
    return {"small_batch": {
        "workload": f"the first 64 / 256 tokens of the step's inputs (H={H}, E={E}, k={K}); "
                    "route, map (one launch), FP8 expand, combine",
        "timing": "HIP graph of the steps", "launches_per_step": 4, **res}}


def bench_quant(tk, torch, x, steps):
    """Each codec granularity on the step's hidden states (8192 x 7168 bf16)."""
    out = {}
    names = {tk.TK_QUANT_FP8_1X128: "quant_fp8_1x128", tk.TK_QUANT_FP8_1X128_POW2: "quant_fp8_1x128_pow2",
             tk.TK_QUANT_FP8_128X128: "quant_fp8_128x128",
             tk.TK_QUANT_FP8_PER_CHANNEL: "quant_fp8_per_channel",
             tk.TK_QUANT_FP4_1X32: "quant_fp4_1x32"}
    for mode, name in names.items():
        q, s = tk.tk_quant(x, mode)
        need = int(tk.library().tk_quant_workspace_bytes(T, H, mode))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device) if need else None
        us = _time_calls(torch, lambda: tk.tk_quant(x, mode, q, s, ws), min(steps, 20), (q, s))
        nbytes = T * H * 2 + q.numel() + s.numel() * 4
        if mode == tk.TK_QUANT_FP8_PER_CHANNEL:
            nbytes += T * H * 2          # two passes over x: column maxima, then codes
        out[name] = {"workload": f"x bf16 ({T}, {H})", "us_per_call": round(us, 2),
                     "timing": "HIP graph of the calls",
                     "roofline": {"bound": "hbm", "achieved": round(nbytes / us / 1e3, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(nbytes / us / 1e3 / PEAK_HBM_GBPS, 4),
                                  "algorithmic_bytes": nbytes}}
    return out


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip timing the CPU oracle")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the routing path is built and timed on a single "
              "MI355X; runs on more than one GPU are not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from __graft_entry__ import _ensure_built
    _ensure_built()
    import moe_routing_amd as tk
    from moe_routing_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    gate = synth.v3_gate(0)
    r = gate["route"]
    x_h = synth.v3_hidden(0)
    y_h = synth.v3_expert_out(0, R, H)

    def up(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if bf16 else a)).to(dev)
        return t.view(torch.bfloat16) if bf16 else t

    logits, bias = up(gate["logits"]), up(gate["bias"])
    x, y = up(x_h, True), up(y_h, True)
    opts = tk.RouteOpts(**r)
    idx = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    pos = torch.empty((T, K), dtype=torch.int32, device=dev)
    row_src = torch.empty(R, dtype=torch.int32, device=dev)
    ws = torch.empty(max(tk.tk_map_workspace_bytes(T, K, E), 4), dtype=torch.uint8, device=dev)
    xq = torch.empty((R, H), dtype=torch.uint8, device=dev)
    sc = torch.empty((R, NB), dtype=torch.float32, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    steps = ("route", "map", "expand", "reduce")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        tk.tk_route(logits, bias, K, opts, idx, w)
        if ev is not None:
            ev[1].record()
        tk.tk_map(idx, E, 0, E, counts, offsets, pos, row_src, ws)
        if ev is not None:
            ev[2].record()
        tk.tk_expand_quant(x, pos, tk.TK_EXPAND_FP8_E4M3_1X128, R, xq, sc)
        if ev is not None:
            ev[3].record()
        tk.tk_reduce_dense(y, pos, w, out)
        if ev is not None:
            ev[4].record()

    _progress(f"inputs resident; {args.warmup} warm-up passes")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Headline: `steps` passes, each started with the MALL (256 MB) and the
    # L2s evicted by a 1 GiB read, so no input of the step is cached when it
    # starts (a read, not a write: a write would leave up to 256 MB of dirty
    # lines whose write-back the timed step would pay for; the read also
    # drains the previous pass's own dirty lines).  Each pass is timed by one
    # pair of HIP events on the launch stream (torch's current stream, which
    # every tk_* call uses), with the host synchronised before and after; no
    # event sits between the kernels.
    flush = torch.ones(1 << 28, dtype=torch.int32, device=dev)
    ev_a = torch.cuda.Event(enable_timing=True)
    ev_b = torch.cuda.Event(enable_timing=True)
    cold = []
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        flush.sum()
        ev_a.record()
        step()
        ev_b.record()
        torch.cuda.synchronize()
        cold.append(ev_a.elapsed_time(ev_b))
    wall_cold = time.perf_counter() - wall0
    _progress(f"{args.steps} flushed passes: {sum(cold) / len(cold) * 1e3:.1f} us per pass")

    # Warm: the same number of passes back to back between two events (x
    # stays in the MALL from one pass to the next, so this is faster).
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev_a.record()
    for _ in range(args.steps):
        step()
    ev_b.record()
    torch.cuda.synchronize()
    wall_warm = time.perf_counter() - wall0
    warm_ms = ev_a.elapsed_time(ev_b) / args.steps
    _progress(f"{args.steps} back-to-back passes: {warm_ms * 1e3:.1f} us per pass")

    # Per-kernel breakdown: passes with an event between consecutive calls,
    # back to back and after a flush; the roofline of the dominant kernel
    # comes from the back-to-back pass.
    def breakdown(n, flushed):
        per = {s: [] for s in steps}
        for _ in range(n):
            if flushed:
                flush.sum()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
            step(ev)
            if flushed:
                torch.cuda.synchronize()
                for j, s in enumerate(steps):
                    per[s].append(ev[j].elapsed_time(ev[j + 1]))
            else:
                evs.append(ev)
        return per

    evs = []
    breakdown(args.steps, False)
    torch.cuda.synchronize()
    per = {s: [] for s in steps}
    for e in evs:
        for j, s in enumerate(steps):
            per[s].append(e[j].elapsed_time(e[j + 1]))
    kern_us = {s: 1e3 * float(np.mean(v)) for s, v in per.items()}
    kern_med_us = {s: 1e3 * float(np.median(v)) for s, v in per.items()}
    kern_p10_us = {s: 1e3 * float(np.percentile(v, 10)) for s, v in per.items()}
    kern_p90_us = {s: 1e3 * float(np.percentile(v, 90)) for s, v in per.items()}
    cold_per = breakdown(min(args.steps, 10), True)
    cold_kern_us = {s: 1e3 * float(np.median(v)) for s, v in cold_per.items()}
    del flush

    # The last flushed pass's outputs, for the comparison with the oracle.
    step()
    torch.cuda.synchronize()
    gpu_out = {"idx": idx.cpu().numpy(), "w": w.cpu().numpy(), "counts": counts.cpu().numpy(),
               "offsets": offsets.cpu().numpy(), "pos": pos.cpu().numpy(),
               "row_src": row_src.cpu().numpy(), "xq": xq.cpu().numpy(), "sc": sc.cpu().numpy(),
               "out": out.view(torch.int16).cpu().numpy().view(np.uint16)}
    copy_gbps = stream_copy_gbps(torch, dev)

    if args.calib_copy:
        # a plain device copy of known size, for scaling the HBM byte counters
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    _progress("breakdown passes done; timing the next rows")
    next_rows = {"swiglu_quant_fp8": bench_swiglu(tk, torch, y, offsets[E:], row_src, pos, w,
                                                  args.steps),
                 **bench_map_balance(tk, torch, logits, idx, args.steps),
                 **bench_quant(tk, torch, x, args.steps),
                 **bench_expand_bf16(tk, torch, x, pos, args.steps),
                 **bench_combines(tk, torch, y, pos, w, args.steps),
                 **bench_ep_share(tk, torch, np, synth, dev, args.steps),
                 **bench_small_batch(tk, torch, logits, bias, x, y, opts, args.steps)}

    ms_per_step = float(np.mean(cold))
    value = T / (ms_per_step * 1e-3)
    gbps = BYTES["total"] / (ms_per_step * 1e-3) / 1e9
    warm_gbps = BYTES["total"] / (warm_ms * 1e-3) / 1e9
    # tk_reduce_dense runs rounds of one 16-token workgroup per CU, each round
    # a launch of its own when a round moves at least 480 MiB (at this shape
    # on 256 CUs: two launches of 4096 tokens); the roofline is per launch: a
    # launch's share of the bytes over its share of the call's time
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    rounds = -(-(-(-T // 16)) // cus)
    round_bytes = cus * 16 * ((2 * K + 2) * H + 8 * K)
    red_launches = rounds if round_bytes >= (480 << 20) else 1
    red_s = kern_us["reduce"] * 1e-6 / red_launches
    achieved = BYTES["reduce"] / red_launches / red_s / 1e9
    traffic = measured_traffic()
    result = {
        "metric": "routed tokens/s and achieved HBM GB/s (% of peak), T=8192 H=7168 E=256 k=8",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 gating / e4m3 dispatch / bf16 combine (fp32 acc)",
        "data": "synthetic",
        "config": {"workload": WORKLOAD, "T": T, "H": H, "E": E, "k": K, "n_groups": 8,
                   "topk_groups": 4, "route_scale": 2.5, "global_batch": T,
                   "io": "logits fp32, hidden bf16, dispatch E4M3 + fp32 scales, combine bf16",
                   "parallelism": "single GPU"},
        "timing": "each timed pass starts with the MALL and L2 evicted (1 GiB device read) and "
                  "is bracketed by one pair of HIP events on the launch stream; value and "
                  "ms_per_step are the mean over the passes",
        "hbm_gbps": round(gbps, 1),
        "hbm_frac": round(gbps / PEAK_HBM_GBPS, 4),
        "hbm_frac_cold": round(gbps / PEAK_HBM_GBPS, 4),
        "ms_per_step_cold_median": round(float(np.median(cold)), 5),
        "ms_per_step_cold_p10_p90": [round(float(np.percentile(cold, 10)), 5),
                                     round(float(np.percentile(cold, 90)), 5)],
        "algorithmic_bytes_per_step": BYTES["total"],
        "warm": {"ms_per_step": round(warm_ms, 5), "tokens_per_s": round(T / (warm_ms * 1e-3), 1),
                 "hbm_gbps": round(warm_gbps, 1), "hbm_frac": round(warm_gbps / PEAK_HBM_GBPS, 4),
                 "timing": "the same passes back to back between two events: x stays in the "
                           "MALL from one pass to the next"},
        "kernel_us_mean": {s: round(v, 2) for s, v in kern_us.items()},
        "kernel_us_median": {s: round(v, 2) for s, v in kern_med_us.items()},
        "kernel_us_p10": {s: round(v, 2) for s, v in kern_p10_us.items()},
        "kernel_us_p90": {s: round(v, 2) for s, v in kern_p90_us.items()},
        "kernel_us_median_cold": {s: round(v, 2) for s, v in cold_kern_us.items()},
        "kernel_breakdown": "further passes with an event between calls (each event record "
                            "adds a few microseconds): back to back, and after a flush (_cold)",
        "stream_copy": None if copy_gbps is None else {
            "gbps": round(copy_gbps, 1),
            "what": "in-repository streaming copy kernel (libtk_calib.so), 1 GiB, read + written "
                    "bytes over time",
            "pipeline_frac_of_copy": round(gbps / copy_gbps, 4),
            "warm_pipeline_frac_of_copy": round(warm_gbps / copy_gbps, 4)},
        "kernel_gbps": {s: round(BYTES[s] / (kern_us[s] * 1e-6) / 1e9, 1) for s in steps},
        "wall_s_timed": round(wall_cold, 4),
        "wall_s_warm": round(wall_warm, 4),
        "roofline": {"kernel": "reduce_staged_kernel<8>", "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": BYTES["reduce"] // red_launches,
                     "launches_per_call": red_launches,
                     "launch_us": round(kern_us["reduce"] / red_launches, 2)},
        "parity": None,
        "cpu_baseline": None,
        "next_rows": next_rows,
    }
    rc = 0
    if not args.no_cpu_baseline:
        _progress("next rows done; running the CPU oracle on the step's inputs")
        inputs = (gate["logits"], gate["bias"], x_h, y_h, r)
        result["cpu_baseline"], ref = cpu_baseline(inputs)
        result["parity"] = step_parity(gpu_out, ref)
        rc = 0 if result["parity"]["ok"] else 1
    print(json.dumps(result), flush=True)
    if rc:
        print("bench.py: the step's GPU outputs do not match the oracle (see parity)",
              file=sys.stderr)
    return rc


if __name__ == "__main__":
    sys.exit(main())
