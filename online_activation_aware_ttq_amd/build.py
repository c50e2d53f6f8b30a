"""Build the gfx950 TTQ library (``libttq.so``) in-tree with hipcc.

Usage: ``python -m online_activation_aware_ttq_amd.build [-v]``.

Every HIP translation unit is compiled with
  * ``--offload-arch=gfx950`` (MI355X, CDNA4),
  * ``-ffp-contract=off``: the code decision is a fixed float32 sequence and
    must not be fused into multiply-adds (the kernels write ``fmaf`` where a
    fused multiply-add is wanted),
  * ``-Xclang -target-feature -Xclang -packed-fp32-ops``: no packed fp32
    VALU instructions are generated.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libttq.so")

SOURCES = [
    "k_stats.hip",
    "k_fused.hip",
    "k_quant.hip",
    "k_gemm.hip",
    "k_gemm_lds.hip",
    "k_lowrank.hip",
    "k_gemv.hip",
    "k_qgemv.hip",
    "k_qfused.hip",
    "k_gemm_q.hip",
    "k_segment.hip",
    "k_pca.hip",
    "k_stream.hip",
    "ttq_api.cpp",
]

ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-variable",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libttq.so)")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if verbose or res.returncode != 0:
        out = (res.stdout + res.stderr).strip()
        # the host pass does not know the gfx feature flag; that note is noise
        out = "\n".join(x for x in out.splitlines()
                        if "packed-fp32-ops" not in x)
        if out:
            print(out, file=sys.stderr)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}")
    return obj


def build(verbose: bool = False, jobs: int = 6) -> str:
    """Compile all sources and link ``libttq.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    # every symbol must resolve at link time (a kernel whose host stub the
    # compiler did not emit would otherwise fail only when first launched)
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Wl,--no-undefined", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        print(res.stdout + res.stderr, file=sys.stderr)
        raise RuntimeError("linking libttq.so failed")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def build_host_sanitized(out_dir: str, verbose: bool = False) -> str:
    """``libttq.so`` with the host layer (``ttq_api.cpp``: validation,
    planning, workspace offsets) built with AddressSanitizer and
    UndefinedBehaviorSanitizer, linked with the kernel objects of the regular
    build (``build()`` first).  Loaded through ``TTQ_LIBRARY`` with the ASan
    runtime preloaded (``asan_runtime()``); only host code is instrumented."""
    objs = [os.path.join(BUILD_DIR, s + ".o") for s in SOURCES if s != "ttq_api.cpp"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError(f"kernel objects missing ({missing[0]}): run build() first")
    os.makedirs(out_dir, exist_ok=True)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(out_dir, "ttq_api_san.o")
    flags = [f for f in COMMON_FLAGS if f != "-O3"] + ["-O1", "-g"]
    cmd = [_hipcc(), "-x", "hip", *flags, *san, "-c",
           os.path.join(CSRC, "ttq_api.cpp"), "-o", api_obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        print(res.stdout + res.stderr, file=sys.stderr)
        raise RuntimeError("hipcc failed on the sanitized ttq_api.cpp")
    lib = os.path.join(out_dir, "libttq.so")
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", lib,
           api_obj, *objs, *san[:4], "-shared-libsan"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        print(res.stdout + res.stderr, file=sys.stderr)
        raise RuntimeError("linking the sanitized libttq.so failed")
    return lib


def asan_runtime() -> str:
    """Path of the clang ASan runtime that a sanitized build needs preloaded."""
    out = subprocess.run([_hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True).stdout.strip()
    if out and os.path.exists(out):
        return out
    import glob
    cands = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not cands:
        raise RuntimeError("the ASan runtime (libclang_rt.asan-x86_64.so) was not found")
    return cands[0]


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
