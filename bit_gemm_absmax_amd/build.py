"""Builds libbitlinear.so (HIP, gfx950) in-tree with hipcc, and beside it
libblbench.so, the benchmark's streaming-read reference kernel (csrc/bench;
measurement support, not part of the BitLinear path).

Usage: ``python -m bit_gemm_absmax_amd.build`` or :func:`build` from Python.
Every call recompiles all sources.  ``build_sanitized()`` (``--sanitize``)
builds a separate copy whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer (device code unchanged) under _build/sanitize/,
for host-side checks on a machine without a GPU.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libbitlinear.so")
BENCH_LIB = os.path.join(PKG, "libblbench.so")
BENCH_SRC = os.path.join(CSRC, "bench")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: epilogue arithmetic must be separate IEEE operations.
# -fhip-fp32-correctly-rounded-divide-sqrt: 127/gamma and W/gamma are IEEE divides.
# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
# -amdgpu-kernarg-preload-count: the first kernel arguments (as many as the
#   free user SGPRs hold, 32 bytes here) are preloaded into SGPRs at wave
#   launch, so a kernel's first loads need not wait for an argument fetch;
#   firmware without the feature runs the compiler's fallback block that
#   loads them as before.  Decode step at M=1 8.20 -> 7.67 us.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    "-Wall", "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Host-only sanitizers: each -fsanitize= applies to the host pass alone.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_DIR = os.path.join(BUILD_DIR, "sanitize")
SAN_LIB = os.path.join(SAN_DIR, "libbitlinear.so")


def _compile(src: str, extra=(), out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    # dlopen resolves every symbol now: a kernel whose host stub the
    # compiler failed to emit shows up here, at build time, not at first use.
    import ctypes
    ctypes.CDLL(tmp)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    bench_srcs = sorted(os.path.join(BENCH_SRC, f) for f in os.listdir(BENCH_SRC) if f.endswith(".hip"))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(bench_srcs))) as ex:
        objs = list(ex.map(_compile, srcs + bench_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], BENCH_LIB)
    if verbose:
        print(f"built {LIB}")
        print(f"built {BENCH_LIB}")
    return LIB


def build_sanitized(verbose: bool = False) -> str:
    """libbitlinear with host-side ASan + UBSan in _build/sanitize/ (load it
    with the clang ASan runtime preloaded)."""
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, SAN_FLAGS, SAN_DIR), srcs))
    tmp = SAN_LIB + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    if verbose:
        print(f"built {SAN_LIB}")
    return SAN_LIB


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
