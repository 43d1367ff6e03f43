"""Build libtk.so (the HIP C-ABI library) in-tree for gfx950.

First a host-only generator (sigmoid_table_gen.hip) is compiled and run: it
writes _build/sigmoid_table.inc, the pinned sigmoid at every bf16 value of
its band, which swiglu.hip includes.  Then each .hip source is compiled to an
object under _build/ in parallel and linked into moe_routing_amd/libtk.so;
calib.hip (a streaming copy bench.py measures for reference) becomes
moe_routing_amd/libtk_calib.so.
Always recompiles (a build check must compile); callers that only need the
library load it when it exists.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libtk.so")
CALIB_LIB = os.path.join(PKG, "libtk_calib.so")   # bench.py's stream-copy reference
SOURCES = ["api.hip", "route.hip", "map.hip", "expand.hip", "reduce.hip", "swiglu.hip", "balance.hip", "quant.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -ffp-contract=off: every fp32 step written in the kernels is one IEEE op
#   (the pinned sigmoid and the Markstein quotient depend on it);
# correctly rounded fp32 division and sqrt, denormals kept (IEEE mode);
# packed-fp32 instructions disabled for the whole device build.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC, "-I", BUILD,
]


def _sigmoid_table() -> None:
    exe = os.path.join(BUILD, "sigmoid_table_gen")
    cmd = [HIPCC, "--cuda-host-only", "-O2", "-std=c++17", "-ffp-contract=off", "-I", INCLUDE,
           "-I", CSRC, os.path.join(CSRC, "sigmoid_table_gen.hip"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on sigmoid_table_gen.hip:\n{r.stdout}\n{r.stderr}")
    r = subprocess.run([exe, os.path.join(BUILD, "sigmoid_table.inc")], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sigmoid_table_gen failed:\n{r.stdout}\n{r.stderr}")


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _sigmoid_table()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    obj = _compile("calib.hip")
    tmp = CALIB_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", obj, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (calib):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
