"""Scalar CPU oracle for the BitNet b1.58 BitLinear layer (W1.58A8).

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check in the package
entry module and the CPU-baseline leg of the benchmark may import this module;
the product path (HIP library and its binding) never does, and the two share
no code.

The arithmetic lives in ``oracle.c`` (plain C, built with gcc); this module
only builds it, loads it and marshals numpy arrays.  The C file is built
twice: ``liboracle.so`` runs on one core, ``liboracle_mt.so`` (``-fopenmp``)
splits the outermost loop of each step over threads with the per-element
code unchanged, so it returns identical results (pinned by a test).  Calls go
to the one-core build unless :func:`set_threads` (or :func:`parallel`) asks
for more threads.  Method source: the
transformers documentation page "BitNet", section "Model details"
(Architecture and Quantization bullets) and section "BitNetConfig"
(rms_norm_eps, model shapes).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_LIB_MT = os.path.join(_HERE, "liboracle_mt.so")

CFLAGS = ["-O2", "-fno-tree-vectorize", "-ffp-contract=off", "-fno-fast-math",
          "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra"]
# (extra flags, output) of the two builds of oracle.c
_BUILDS = {"serial": (["-Wno-unknown-pragmas"], _LIB), "mt": (["-fopenmp"], _LIB_MT)}
_CC = "gcc"
# ORACLE_SANITIZE=1: both builds with AddressSanitizer and UndefinedBehaviorSanitizer
# (clang, so one sanitizer runtime serves this and the HIP library's host code),
# under separate names; the arithmetic flags are the same.
if os.environ.get("ORACLE_SANITIZE") == "1":
    _CC = "/opt/rocm/llvm/bin/clang"
    _SAN = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer", "-g"]
    _LIB = os.path.join(_HERE, "liboracle_san.so")
    _LIB_MT = os.path.join(_HERE, "liboracle_mt_san.so")
    _BUILDS = {"serial": (["-Wno-unknown-pragmas", *_SAN], _LIB), "mt": (["-fopenmp", *_SAN], _LIB_MT)}

_libs = {}
_threads = 1


def _compile(which: str) -> str:
    extra, out = _BUILDS[which]
    tmp = out + ".tmp"
    subprocess.run([_CC, *CFLAGS, *extra, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build() -> str:
    """Compile oracle.c into liboracle.so and liboracle_mt.so with gcc (always
    recompiles both)."""
    for which in _BUILDS:
        _compile(which)
    return _LIB


def default_threads() -> int:
    """Host threads for the OpenMP build: OMP_NUM_THREADS if set, else the
    cores this process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux
        return os.cpu_count() or 1


def set_threads(n: int) -> int:
    """Route later calls to the one-core build (n == 1) or to the OpenMP build
    with n threads; returns the thread count in force."""
    global _threads
    n = max(1, int(n))
    if n > 1:
        got = _load("mt").orc_set_threads(n)
        _threads = max(1, int(got))
    else:
        _threads = 1
    return _threads


def threads() -> int:
    return _threads


@contextlib.contextmanager
def parallel(n=None):
    """Run the enclosed oracle calls on the OpenMP build with n threads
    (default: default_threads())."""
    prev = _threads
    set_threads(default_threads() if n is None else n)
    try:
        yield _threads
    finally:
        set_threads(prev)


def _load(which: str = None):
    if which is None:
        which = "mt" if _threads > 1 else "serial"
    if which in _libs:
        return _libs[which]
    path = _BUILDS[which][1]
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(_SRC):
        _compile(which)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    F = ctypes.c_float
    lib.orc_absmean_scale.argtypes = [P, I64, I64]
    lib.orc_absmean_scale.restype = F
    lib.orc_ternarize.argtypes = [P, I64, I64, F, P]
    lib.orc_ternarize.restype = None
    lib.orc_pack.argtypes = [P, I64, I64, P]
    lib.orc_pack.restype = ctypes.c_int
    lib.orc_unpack.argtypes = [P, I64, I64, P]
    lib.orc_unpack.restype = ctypes.c_int
    lib.orc_quant_act.argtypes = [P, I64, I64, P, P, P]
    lib.orc_quant_act.restype = None
    lib.orc_rmsnorm.argtypes = [P, I64, I64, P, F, P]
    lib.orc_rmsnorm.restype = None
    lib.orc_int_matmul.argtypes = [P, I64, I64, P, I64, P]
    lib.orc_int_matmul.restype = None
    lib.orc_dequant.argtypes = [P, I64, I64, P, F, P]
    lib.orc_dequant.restype = None
    lib.orc_relu2.argtypes = [P, I64]
    lib.orc_relu2.restype = None
    lib.orc_add.argtypes = [P, P, I64]
    lib.orc_add.restype = None
    lib.orc_ffn_layer.argtypes = [P, I64, I64, I64, P, F, P, F, P, F, P, F,
                                  ctypes.c_int, P, P, P]
    lib.orc_mul.argtypes = [P, P, I64]
    lib.orc_mul.restype = None
    lib.orc_ffn_layer_gated.argtypes = [P, I64, I64, I64, P, F, P, F, P, F, P, F, P, F, ctypes.c_int, P, P, P]
    lib.orc_ffn_layer_gated.restype = None
    lib.orc_ffn_layer.restype = None
    lib.orc_pack_canonical.argtypes = [P, I64, I64, P]
    lib.orc_pack_canonical.restype = ctypes.c_int
    lib.orc_unpack_canonical.argtypes = [P, I64, I64, P]
    lib.orc_unpack_canonical.restype = ctypes.c_int
    lib.orc_set_threads.argtypes = [ctypes.c_int]
    lib.orc_set_threads.restype = ctypes.c_int
    _libs[which] = lib
    return lib


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


RMS_EPS = 1e-5  # "BitNetConfig": rms_norm_eps default


def absmean_scale(W) -> np.float32:
    """Per-tensor absmean of W [N][K] (binary64 sum, one rounding), floored at 1e-5."""
    W = _c(W, np.float32)
    N, K = W.shape
    return np.float32(_load().orc_absmean_scale(_p(W), N, K))


def ternarize(W, gamma) -> np.ndarray:
    """q = clamp(rint(W / gamma), -1, 1) as int8 [N][K]."""
    W = _c(W, np.float32)
    N, K = W.shape
    q = np.empty((N, K), np.int8)
    _load().orc_ternarize(_p(W), N, K, float(np.float32(gamma)), _p(q))
    return q


def quantize_weights(W):
    """Absmean ternarisation: returns (q int8 [N][K], gamma_w float32)."""
    g = absmean_scale(W)
    return ternarize(W, g), g


def pack(q) -> np.ndarray:
    """2-bit encoding of ternary q [N][K] -> N*K/4 bytes, shaped [N][K/4] (the
    bytes are grouped by 16-row tiles, not by row: layout in oracle.h)."""
    q = _c(q, np.int8)
    N, K = q.shape
    out = np.empty((N, K // 4), np.uint8)
    if _load().orc_pack(_p(q), N, K, _p(out)) != 0:
        raise ValueError("pack: K must be a multiple of 64 and q ternary")
    return out


def unpack(packed, K) -> np.ndarray:
    packed = _c(packed, np.uint8)
    N = packed.shape[0]
    q = np.empty((N, K), np.int8)
    if _load().orc_unpack(_p(packed), N, K, _p(q)) != 0:
        raise ValueError("unpack: bad K or code 3 present")
    return q


def pack_canonical(q) -> np.ndarray:
    """Plain 2-bit form of ternary q [N][K]: row-major [N][K/4] bytes, weight
    k in byte k/4 at bits 2(k%4), code q + 1 (orc_pack_canonical)."""
    q = _c(q, np.int8)
    N, K = q.shape
    out = np.empty((N, K // 4), np.uint8)
    if _load().orc_pack_canonical(_p(q), N, K, _p(out)) != 0:
        raise ValueError("pack_canonical: K must be a multiple of 4 and q ternary")
    return out


def unpack_canonical(b, K) -> np.ndarray:
    b = _c(b, np.uint8)
    N = b.shape[0]
    q = np.empty((N, K), np.int8)
    if _load().orc_unpack_canonical(_p(b), N, K, _p(q)) != 0:
        raise ValueError("unpack_canonical: bad K or code 3 present")
    return q


def quant_act(X):
    """Per-token absmax int8: returns (xq int8 [M][K], gamma_x f32 [M], rowsum i32 [M])."""
    X = _c(X, np.float32)
    M, K = X.shape
    xq = np.empty((M, K), np.int8)
    g = np.empty(M, np.float32)
    rs = np.empty(M, np.int32)
    _load().orc_quant_act(_p(X), M, K, _p(xq), _p(g), _p(rs))
    return xq, g, rs


def rmsnorm(V, gain=None, eps=RMS_EPS) -> np.ndarray:
    V = _c(V, np.float32)
    M, K = V.shape
    gain = None if gain is None else _c(gain, np.float32)
    Z = np.empty((M, K), np.float32)
    _load().orc_rmsnorm(_p(V), M, K, _p(gain), float(np.float32(eps)), _p(Z))
    return Z


def int_matmul(xq, q) -> np.ndarray:
    """acc[m][n] = sum_k xq[m][k] * q[n][k] (int32)."""
    xq = _c(xq, np.int8)
    q = _c(q, np.int8)
    M, K = xq.shape
    N, K2 = q.shape
    assert K == K2
    acc = np.empty((M, N), np.int32)
    _load().orc_int_matmul(_p(xq), M, K, _p(q), N, _p(acc))
    return acc


def dequant(acc, gamma_x, gamma_w) -> np.ndarray:
    acc = _c(acc, np.int32)
    gx = _c(gamma_x, np.float32)
    M, N = acc.shape
    Y = np.empty((M, N), np.float32)
    _load().orc_dequant(_p(acc), M, N, _p(gx), float(np.float32(gamma_w)), _p(Y))
    return Y


def relu2(Y) -> np.ndarray:
    Y = np.array(Y, dtype=np.float32, copy=True, order="C")
    _load().orc_relu2(_p(Y), Y.size)
    return Y


def add(H, Y) -> np.ndarray:
    H = np.array(H, dtype=np.float32, copy=True, order="C")
    Y = _c(Y, np.float32)
    assert H.shape == Y.shape
    _load().orc_add(_p(H), _p(Y), H.size)
    return H


def bitlinear(X, q, gamma_w, relu_sq=False):
    """One BitLinear: absmax-quant X, contract with ternary q, dequantise.

    Returns dict with xq, gamma_x, rowsum, acc, y."""
    xq, gx, rs = quant_act(X)
    acc = int_matmul(xq, q)
    y = dequant(acc, gx, gamma_w)
    if relu_sq:
        y = relu2(y)
    return {"xq": xq, "gamma_x": gx, "rowsum": rs, "acc": acc, "y": y}


def ffn_layer(H, q_up, gamma_up, q_down, gamma_down, pre_gain=None,
              sub_gain=None, residual=True, eps=RMS_EPS, intermediates=False):
    """One BitNet FFN block (see orc_ffn_layer).  H [M][Hd] is not modified.

    With pre_gain None the pre-norm is skipped; sub_gain None means unit gain."""
    H = np.array(H, dtype=np.float32, copy=True, order="C")
    M, Hd = H.shape
    q_up = _c(q_up, np.int8)
    q_down = _c(q_down, np.int8)
    F = q_up.shape[0]
    assert q_up.shape == (F, Hd) and q_down.shape == (Hd, F)
    pg = None if pre_gain is None else _c(pre_gain, np.float32)
    sg = _c(np.ones(F, np.float32) if sub_gain is None else sub_gain, np.float32)
    y1 = np.empty((M, F), np.float32) if intermediates else None
    xq2 = np.empty((M, F), np.int8) if intermediates else None
    g2 = np.empty(M, np.float32) if intermediates else None
    _load().orc_ffn_layer(_p(H), M, Hd, F, _p(pg), float(np.float32(eps)),
                          _p(q_up), float(np.float32(gamma_up)), _p(sg),
                          float(np.float32(eps)), _p(q_down),
                          float(np.float32(gamma_down)), int(bool(residual)),
                          _p(y1), _p(xq2), _p(g2))
    if intermediates:
        return H, {"y1": y1, "xq2": xq2, "g2": g2}
    return H


def mul(A, B) -> np.ndarray:
    """Elementwise product in binary32 (orc_mul)."""
    A = np.array(A, dtype=np.float32, copy=True, order="C")
    B = _c(B, np.float32)
    assert A.shape == B.shape
    _load().orc_mul(_p(A), _p(B), A.size)
    return A


def ffn_layer_gated(H, q_gate, gamma_gate, q_up, gamma_up, q_down, gamma_down, pre_gain=None,
                    sub_gain=None, residual=True, eps=RMS_EPS, intermediates=False):
    """One gated BitNet FFN block (see orc_ffn_layer_gated): h =
    ReLU^2(gate) * up, then subln, requantisation and down.  H is not
    modified; intermediates returns h as "y1"."""
    H = np.array(H, dtype=np.float32, copy=True, order="C")
    M, Hd = H.shape
    q_gate = _c(q_gate, np.int8)
    q_up = _c(q_up, np.int8)
    q_down = _c(q_down, np.int8)
    F = q_up.shape[0]
    assert q_gate.shape == (F, Hd) and q_up.shape == (F, Hd) and q_down.shape == (Hd, F)
    pg = None if pre_gain is None else _c(pre_gain, np.float32)
    sg = _c(np.ones(F, np.float32) if sub_gain is None else sub_gain, np.float32)
    y1 = np.empty((M, F), np.float32) if intermediates else None
    xq2 = np.empty((M, F), np.int8) if intermediates else None
    g2 = np.empty(M, np.float32) if intermediates else None
    _load().orc_ffn_layer_gated(_p(H), M, Hd, F, _p(pg), float(np.float32(eps)),
                                _p(q_gate), float(np.float32(gamma_gate)),
                                _p(q_up), float(np.float32(gamma_up)), _p(sg),
                                float(np.float32(eps)), _p(q_down),
                                float(np.float32(gamma_down)), int(bool(residual)),
                                _p(y1), _p(xq2), _p(g2))
    if intermediates:
        return H, {"y1": y1, "xq2": xq2, "g2": g2}
    return H


def ffn_stack(H, layers, residual=True, eps=RMS_EPS):
    """Apply a list of layer dicts (q_up, gamma_up, q_down, gamma_down,
    pre_gain, sub_gain) in order."""
    for L in layers:
        H = ffn_layer(H, L["q_up"], L["gamma_up"], L["q_down"], L["gamma_down"],
                      pre_gain=L.get("pre_gain"), sub_gain=L.get("sub_gain"),
                      residual=residual, eps=eps)
    return H
