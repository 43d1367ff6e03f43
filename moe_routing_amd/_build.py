"""Build libtk.so (the HIP C-ABI library) in-tree for gfx950.

First a host-only generator (sigmoid_table_gen.hip) is compiled and run: it
writes _build/sigmoid_table.inc, the pinned sigmoid at every bf16 value of
its band, which swiglu.hip includes.  Then each .hip source is compiled to an
object under _build/ in parallel and linked into moe_routing_amd/libtk.so;
calib.hip (a streaming copy bench.py measures for reference) becomes
moe_routing_amd/libtk_calib.so.  build_asan() builds the same library with
AddressSanitizer on the host side only (argument checks, error state, launch
wrappers; the device code is built as usual) into _build/asan/, for the CPU
test that runs the boundary checks under the ASan runtime.
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


ASAN_DIR = os.path.join(BUILD, "asan")
ASAN_LIB = os.path.join(ASAN_DIR, "libtk_host_asan.so")
# AddressSanitizer for the host code only: each -fsanitize= goes to the host
# compilation (-Xarch_host), never to the gfx950 device code.
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
              "-Xarch_host", "-g"]


def asan_runtime() -> str | None:
    """Path of the compiler's shared ASan runtime, or None."""
    r = subprocess.run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def _compile(src: str, out_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
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


def build_asan(verbose: bool = False) -> str:
    """libtk with AddressSanitizer on the host code, in _build/asan/ (not loaded
    by the package; the ASan CPU test loads it under the ASan runtime)."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    if not os.path.exists(os.path.join(BUILD, "sigmoid_table.inc")):
        _sigmoid_table()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, ASAN_DIR, ASAN_FLAGS), SOURCES))
    tmp = ASAN_LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *ASAN_FLAGS,
           "-Xarch_host", "-shared-libasan", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (asan):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ASAN_LIB)
    if verbose:
        print(f"built {ASAN_LIB}")
    return ASAN_LIB


ABI_PIPELINE_SRC = os.path.join(ROOT, "tests", "helpers", "abi_pipeline.c")
ABI_PIPELINE = os.path.join(ROOT, "tests", "helpers", "abi_pipeline")


def build_abi_pipeline(verbose: bool = False) -> str:
    """The C program the GPU tests run to drive the routing path through the C
    ABI alone (tests/helpers/abi_pipeline.c): plain C11 with the host
    compiler, linked against libtk.so and the HIP runtime, found at run time
    relative to the program."""
    rocm = os.path.dirname(os.path.dirname(HIPCC))
    tmp = ABI_PIPELINE + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-isystem", os.path.join(rocm, "include"),
           ABI_PIPELINE_SRC, "-o", tmp, "-L", PKG, "-ltk", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../moe_routing_amd",
           f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"gcc failed on abi_pipeline.c:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, ABI_PIPELINE)
    if verbose:
        print(f"built {ABI_PIPELINE}")
    return ABI_PIPELINE


if __name__ == "__main__":
    build(verbose=True)
