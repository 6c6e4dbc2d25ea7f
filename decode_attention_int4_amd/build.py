"""Builds librq.so (the HIP library behind include/rq.h) in-tree for gfx950.

    python -m decode_attention_int4_amd.build
    python -m decode_attention_int4_amd.build --sanitize

Each translation unit is compiled separately (in parallel) and linked with
hipcc.  Packed-FP32 instruction selection is disabled for all device code.

--sanitize builds librq_san.so instead: the host side (argument checking,
layout arithmetic, launch setup) under AddressSanitizer and
UndefinedBehaviorSanitizer, device code unchanged (every sanitizer flag is
host-only).  It is for CPU test runs: load it with RQ_LIB=<path> and the
clang ASan runtime preloaded, e.g.

    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang -print-file-name=libclang_rt.asan-x86_64.so) \
    ASAN_OPTIONS=detect_leaks=0 RQ_LIB=decode_attention_int4_amd/librq_san.so \
    ORACLE_LIB=oracle/liboracle_san.so python -m pytest tests -m "not gpu"
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librq.so")
SAN_BUILD = os.path.join(PKG, "_build_san")
SAN_LIB = os.path.join(PKG, "librq_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
             "-Xarch_host", "-shared-libasan"]
SOURCES = ["rq_api.hip", "rq_quant.hip", "rq_decode.hip", "rq_gqa.hip", "rq_bf16.hip",
           "rq_reconstruct.hip"]
HEADERS = ["rq_device.h", "rq_kernels.h", "rq_layout.h", "rq_stage.h"]
ARCH = os.environ.get("RQ_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # one-lane atomics stay single instructions.  The compiler's
    # wave-aggregating rewrite of an atomic (ballot, bit count, then a
    # read-first-lane of the result) waits for the result right after the
    # atomic; the decode kernels' tile claims (an LDS counter, one lane) are
    # read an iteration later, so the plain atomic hides its latency
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


# Per-source flags: the decode kernels are scheduled by LLVM's iterative ILP
# scheduler, which interleaves their matrix ops, code unpacking and LDS reads
# more tightly than the default one (dominant calls 1-3 % faster on MI355X).
# It is not used for the other sources: the compiler crashes on the
# quantize-append source with it.
SOURCE_FLAGS = {
    "rq_decode.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
    "rq_gqa.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(SAN_BUILD if sanitize else BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *(SAN_FLAGS if sanitize else []), "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compiles every source and links librq.so (librq_san.so with the host
    side under ASan + UBSan); returns its path."""
    out = SAN_LIB if sanitize else LIB
    os.makedirs(SAN_BUILD if sanitize else BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda src: _compile(src, sanitize), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}",
           *(SAN_FLAGS if sanitize else []), *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    srcs = [os.path.join(CSRC, s) for s in SOURCES + HEADERS]
    srcs.append(os.path.join(os.path.dirname(PKG), "include", "rq.h"))
    srcs.append(os.path.abspath(__file__))   # compiler flags
    return any(os.path.getmtime(s) > t for s in srcs)


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
    sys.exit(0)
