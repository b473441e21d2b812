"""Host-code sanitizer run (CPU only, no GPU needed).

Builds the HIP library with AddressSanitizer and UndefinedBehaviorSanitizer
on its host code (argument validation, workspace carving, dispatch; the device
code is unchanged) and both oracle builds with the same sanitizers, then runs
the CPU test suite (``-m "not gpu"``) against those builds with the clang
sanitizer runtime preloaded into Python.  Any invalid memory access or
undefined behaviour in the host code or the oracle aborts the run with a
report.  Leak checking is off: the Python interpreter itself is not
instrumented.

Usage:  python tests/sanitize_host.py [extra pytest args]
"""
import glob
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def runtime() -> str:
    libs = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
    if not libs:
        raise SystemExit("clang ASan runtime not found under /opt/rocm/llvm")
    return libs[0]


def main() -> int:
    sys.path.insert(0, ROOT)
    from bit_gemm_absmax_amd import build
    lib = build.build_sanitized(verbose=True)
    env = dict(os.environ)
    env.update({
        "BITLINEAR_LIB": lib,
        "ORACLE_SANITIZE": "1",
        "LD_PRELOAD": runtime(),
        "ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1:halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
    })
    # the oracle's sanitized builds are compiled fresh by the child process
    for name in ("liboracle_san.so", "liboracle_mt_san.so"):
        path = os.path.join(ROOT, "oracle", name)
        if os.path.exists(path):
            os.remove(path)
    cmd = [sys.executable, "-m", "pytest", os.path.join(ROOT, "tests"), "-q", "-m", "not gpu", "-p", "no:cacheprovider",
           *sys.argv[1:]]
    print("+", " ".join(cmd), flush=True)
    return subprocess.run(cmd, env=env, cwd=ROOT).returncode


if __name__ == "__main__":
    sys.exit(main())
