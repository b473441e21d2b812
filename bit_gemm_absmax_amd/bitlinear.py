"""Python binding of libbitlinear (the C ABI in include/bitlinear.h).

Argument marshalling only: every step of the BitLinear path runs in the HIP
kernels of the library.  Tensors are torch CUDA (HIP) tensors; calls enqueue
on torch's current stream and do not synchronise.  If the library is not
built, every call raises :class:`BitLinearError`; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# BITLINEAR_LIB selects another build of the same library (the host-sanitizer
# build of build.py); the default is the in-tree one.
LIB_PATH = os.environ.get("BITLINEAR_LIB") or os.path.join(_HERE, "libbitlinear.so")

BL_OK = 0
BL_ERR_NULL = -1
BL_ERR_SHAPE = -2
BL_ERR_ALIGN = -3
BL_ERR_WORKSPACE = -4
BL_ERR_HIP = -5
BL_ERR_UNSUPPORTED = -6

BL_QUANT_RMSNORM = 0x1
BL_EPI_RELU2 = 0x1
BL_EPI_RESIDUAL = 0x2
BL_EPI_SUBLN_QUANT = 0x4
BL_EPI_MUL = 0x8
BL_FFN_PRE_NORM = 0x1
BL_FFN_RESIDUAL = 0x2
BL_FFN_PERSISTENT = 0x4
BL_DTYPE_F32 = 0
BL_DTYPE_BF16 = 1

RMS_EPS = 1e-5  # rms_norm_eps of the BitNet config

SYMBOLS = (
    "bitlinear_status_string", "bitlinear_last_error", "bitlinear_abi_version",
    "bitlinear_pack_workspace_bytes", "bitlinear_pack_weights",
    "bitlinear_import_canonical", "bitlinear_export_canonical", "bitlinear_unpack_weights",
    "bitlinear_quant_act",
    "bitlinear_forward_workspace_bytes", "bitlinear_forward", "bitlinear_forward_grouped",
    "bitlinear_quant_forward_workspace_bytes", "bitlinear_quant_forward",
    "bitlinear_quant_forward_grouped_workspace_bytes", "bitlinear_quant_forward_grouped",
    "bitlinear_latent_forward_workspace_bytes", "bitlinear_latent_forward",
    "bitnet_ffn_workspace_bytes", "bitnet_ffn_forward", "bitnet_ffn_forward_noalloc",
)
NOALLOC_MAX_BYTES = 64 << 20  # BITNET_FFN_NOALLOC_MAX_BYTES


class BitLinearError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[{status}] {message}")
        self.status = status


class Epilogue(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("residual", ctypes.c_void_p),
                ("norm_gain", ctypes.c_void_p), ("norm_eps", ctypes.c_float),
                ("out_q", ctypes.c_void_p), ("out_q_scale", ctypes.c_void_p),
                ("out_q_rowsum", ctypes.c_void_p), ("mul_by", ctypes.c_void_p)]


BL_MAX_GROUPS = 4


class Group(ctypes.Structure):
    _fields_ = [("packed", ctypes.c_void_p), ("w_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("epi", Epilogue), ("Y", ctypes.c_void_p), ("acc_out", ctypes.c_void_p)]


class FFNLayer(ctypes.Structure):
    _fields_ = [("pre_norm_gain", ctypes.c_void_p), ("up", ctypes.c_void_p),
                ("up_scale", ctypes.c_void_p), ("gate", ctypes.c_void_p),
                ("gate_scale", ctypes.c_void_p), ("sub_norm_gain", ctypes.c_void_p),
                ("down", ctypes.c_void_p), ("down_scale", ctypes.c_void_p)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libbitlinear.so and declare its C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise BitLinearError(BL_ERR_UNSUPPORTED,
                             f"{path} is not built (python -m bit_gemm_absmax_amd.build)")
    lib = ctypes.CDLL(path)
    P, I64, U32, F, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_float, ctypes.c_size_t
    I = ctypes.c_int
    lib.bitlinear_status_string.argtypes = [I]
    lib.bitlinear_status_string.restype = ctypes.c_char_p
    lib.bitlinear_last_error.argtypes = []
    lib.bitlinear_last_error.restype = ctypes.c_char_p
    lib.bitlinear_abi_version.argtypes = []
    lib.bitlinear_abi_version.restype = I
    lib.bitlinear_pack_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_pack_workspace_bytes.restype = SZ
    lib.bitlinear_pack_weights.argtypes = [P, I64, I64, P, P, P, SZ, P]
    lib.bitlinear_pack_weights.restype = I
    for name in ("bitlinear_import_canonical", "bitlinear_export_canonical", "bitlinear_unpack_weights"):
        getattr(lib, name).argtypes = [P, I64, I64, P, P]
        getattr(lib, name).restype = I
    lib.bitlinear_quant_act.argtypes = [P, I64, I64, U32, P, F, P, P, P, P]
    lib.bitlinear_quant_act.restype = I
    lib.bitlinear_forward_workspace_bytes.argtypes = [I64, I64, I64, U32]
    lib.bitlinear_forward_workspace_bytes.restype = SZ
    lib.bitlinear_forward.argtypes = [P, P, P, I64, I64, P, P, I64, ctypes.POINTER(Epilogue),
                                      P, P, P, SZ, P]
    lib.bitlinear_forward.restype = I
    lib.bitlinear_forward_grouped.argtypes = [P, P, P, I64, I64, ctypes.POINTER(Group), ctypes.c_int32, P]
    lib.bitlinear_forward_grouped.restype = I
    lib.bitlinear_quant_forward_grouped_workspace_bytes.argtypes = [I64, I64]
    lib.bitlinear_quant_forward_grouped_workspace_bytes.restype = ctypes.c_size_t
    lib.bitlinear_quant_forward_grouped.argtypes = [P, I64, I64, ctypes.c_uint32, P, ctypes.c_float,
                                                    ctypes.POINTER(Group), ctypes.c_int32, P, ctypes.c_size_t, P]
    lib.bitlinear_quant_forward_grouped.restype = I
    lib.bitlinear_quant_forward_workspace_bytes.argtypes = [I64, I64, I64]
    lib.bitlinear_quant_forward_workspace_bytes.restype = SZ
    lib.bitlinear_quant_forward.argtypes = [P, I64, I64, U32, P, F, P, P, I64, ctypes.POINTER(Epilogue),
                                            P, P, SZ, P]
    lib.bitlinear_quant_forward.restype = I
    lib.bitlinear_latent_forward_workspace_bytes.argtypes = [I64, I64, I64]
    lib.bitlinear_latent_forward_workspace_bytes.restype = SZ
    lib.bitlinear_latent_forward.argtypes = [P, I64, I64, U32, P, F, P, U32, I64, ctypes.POINTER(Epilogue),
                                             P, P, P, SZ, P]
    lib.bitlinear_latent_forward.restype = I
    lib.bitnet_ffn_workspace_bytes.argtypes = [I64, I64, I64]
    lib.bitnet_ffn_workspace_bytes.restype = SZ
    lib.bitnet_ffn_forward.argtypes = [ctypes.POINTER(FFNLayer), ctypes.c_int32, P, I64, I64, I64,
                                       U32, F, P, SZ, P]
    lib.bitnet_ffn_forward.restype = I
    lib.bitnet_ffn_forward_noalloc.argtypes = [ctypes.POINTER(FFNLayer), ctypes.c_int32, P, I64, I64, I64,
                                               U32, F, P]
    lib.bitnet_ffn_forward_noalloc.restype = I
    _lib = lib
    return lib


def _check(status: int):
    if status != BL_OK:
        lib = load()
        msg = lib.bitlinear_last_error().decode() or lib.bitlinear_status_string(status).decode()
        raise BitLinearError(status, msg)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype, ndim: int, name: str):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(*ts):
    """Every given tensor (None skipped) must live on the GPU; checked after
    the dtype and shape checks, right before a call into the library."""
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError(f"a {tuple(t.shape)} {t.dtype} argument is not a GPU tensor")


def _shape(t: Optional[torch.Tensor], dtype, shape, name: str):
    """Exact dtype and shape of an optional tensor argument (the C library
    trusts M, K and N, so a wrong-sized tensor would be read or written past
    its end)."""
    if t is None:
        return
    _need(t, dtype, len(shape), name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return None
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device)


def pack_weights(W: torch.Tensor):
    """Absmean-ternarise and pack fp32 W [N][K] -> (packed u8 [N][K/4], w_scale f32 [1]).

    The packed bytes are grouped by 16-row tiles, not by row (layout in
    include/bitlinear.h): pass the tensor whole; slicing its rows does not give
    the packed form of a row subset."""
    lib = load()
    _need(W, torch.float32, 2, "W")
    _on_gpu(W)
    N, K = W.shape
    packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    w_scale = torch.empty(1, dtype=torch.float32, device=W.device)
    ws = _workspace(lib.bitlinear_pack_workspace_bytes(N, K), W.device)
    _check(lib.bitlinear_pack_weights(_p(W), N, K, _p(packed), _p(w_scale), _p(ws),
                                      0 if ws is None else ws.numel(), _stream(W.device)))
    return packed, w_scale


def _relayout(fn_name: str, src: torch.Tensor, N: int, K: int, out: torch.Tensor):
    lib = load()
    _check(getattr(lib, fn_name)(_p(src), N, K, _p(out), _stream(src.device)))
    return out


def import_canonical(canonical: torch.Tensor) -> torch.Tensor:
    """Plain row-major 2-bit weights u8 [N][K/4] (four consecutive codes q + 1
    per byte, lowest bits first) -> this library's packed layout u8 [N][K/4]."""
    _need(canonical, torch.uint8, 2, "canonical")
    _on_gpu(canonical)
    N, K = canonical.shape[0], canonical.shape[1] * 4
    return _relayout("bitlinear_import_canonical", canonical, N, K,
                     torch.empty_like(canonical))


def export_canonical(packed: torch.Tensor) -> torch.Tensor:
    """The inverse of import_canonical."""
    _need(packed, torch.uint8, 2, "packed")
    _on_gpu(packed)
    N, K = packed.shape[0], packed.shape[1] * 4
    return _relayout("bitlinear_export_canonical", packed, N, K, torch.empty_like(packed))


def unpack_weights(packed: torch.Tensor) -> torch.Tensor:
    """Packed layout u8 [N][K/4] -> ternary q int8 [N][K]."""
    _need(packed, torch.uint8, 2, "packed")
    _on_gpu(packed)
    N, K = packed.shape[0], packed.shape[1] * 4
    return _relayout("bitlinear_unpack_weights", packed, N, K,
                     torch.empty((N, K), dtype=torch.int8, device=packed.device))


def quant_act(X: torch.Tensor, rmsnorm: bool = False, norm_gain: Optional[torch.Tensor] = None,
              eps: float = RMS_EPS, out=None):
    """Per-token absmax int8 of X [M][K] (optionally after RMSNorm) ->
    (Xq int8 [M][K], x_scale f32 [M], x_rowsum i32 [M])."""
    lib = load()
    _need(X, torch.float32, 2, "X")
    M, K = X.shape
    if out is None:
        out = (torch.empty((M, K), dtype=torch.int8, device=X.device),
               torch.empty(M, dtype=torch.float32, device=X.device),
               torch.empty(M, dtype=torch.int32, device=X.device))
    xq, xs, rs = out
    _shape(xq, torch.int8, (M, K), "Xq")
    _shape(xs, torch.float32, (M,), "x_scale")
    _shape(rs, torch.int32, (M,), "x_rowsum")
    _shape(norm_gain, torch.float32, (K,), "norm_gain")
    _on_gpu(X, xq, xs, rs, norm_gain)
    _check(lib.bitlinear_quant_act(_p(X), M, K, BL_QUANT_RMSNORM if rmsnorm else 0, _p(norm_gain),
                                   float(eps), _p(xq), _p(xs), _p(rs), _stream(X.device)))
    return xq, xs, rs


def forward(xq: torch.Tensor, x_scale: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor,
            x_rowsum: Optional[torch.Tensor] = None, relu2: bool = False,
            residual: Optional[torch.Tensor] = None, subln: bool = False,
            norm_gain: Optional[torch.Tensor] = None, eps: float = RMS_EPS,
            want_y: bool = True, want_acc: bool = False, y_out: Optional[torch.Tensor] = None,
            mul_by: Optional[torch.Tensor] = None):
    """BitLinear forward.  Returns a dict with the requested outputs:
    'y' (f32 [M][N]), 'acc' (i32 [M][N]) and, with subln, 'q', 'q_scale', 'q_rowsum'.
    mul_by multiplies the (ReLU^2'd) output elementwise: the gating product."""
    lib = load()
    _need(xq, torch.int8, 2, "xq")
    _need(packed, torch.uint8, 2, "packed")
    M, K = xq.shape
    N = packed.shape[0]
    if packed.shape[1] * 4 != K:
        raise ValueError(f"packed has {packed.shape[1]} bytes per row, expected K/4 = {K // 4}")
    _shape(x_scale, torch.float32, (M,), "x_scale")
    _shape(x_rowsum, torch.int32, (M,), "x_rowsum")
    _shape(w_scale, torch.float32, (1,), "w_scale")
    for t, name in ((residual, "residual"), (mul_by, "mul_by"), (y_out, "y_out")):
        _shape(t, torch.float32, (M, N), name)
    if subln:
        _shape(norm_gain, torch.float32, (N,), "norm_gain")
    _on_gpu(xq, x_scale, x_rowsum, packed, w_scale, residual, mul_by, y_out, norm_gain)
    dev = xq.device
    flags = 0
    epi = Epilogue()
    res = {}
    if relu2:
        flags |= BL_EPI_RELU2
    if residual is not None:
        flags |= BL_EPI_RESIDUAL
        epi.residual = residual.data_ptr()
    if mul_by is not None:
        flags |= BL_EPI_MUL
        epi.mul_by = mul_by.data_ptr()
    if subln:
        flags |= BL_EPI_SUBLN_QUANT
        res["q"] = torch.empty((M, N), dtype=torch.int8, device=dev)
        res["q_scale"] = torch.empty(M, dtype=torch.float32, device=dev)
        res["q_rowsum"] = torch.empty(M, dtype=torch.int32, device=dev)
        epi.out_q = res["q"].data_ptr()
        epi.out_q_scale = res["q_scale"].data_ptr()
        epi.out_q_rowsum = res["q_rowsum"].data_ptr()
        epi.norm_gain = None if norm_gain is None else norm_gain.data_ptr()
        epi.norm_eps = float(eps)
    epi.flags = flags
    y = None
    if want_y or not subln:
        y = y_out if y_out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
        res["y"] = y
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if want_acc else None
    if acc is not None:
        res["acc"] = acc
    ws = _workspace(lib.bitlinear_forward_workspace_bytes(M, K, N, flags), dev)
    _check(lib.bitlinear_forward(_p(xq), _p(x_scale), _p(x_rowsum), M, K, _p(packed), _p(w_scale),
                                 N, ctypes.byref(epi), _p(y), _p(acc), _p(ws),
                                 0 if ws is None else ws.numel(), _stream(dev)))
    return res


def _groups(mats: Sequence[dict], M: int, K: int, dev):
    """The bl_group array and the result dicts of a grouped call."""
    if not 1 <= len(mats) <= BL_MAX_GROUPS:
        raise ValueError(f"1 to {BL_MAX_GROUPS} matrices per call, got {len(mats)}")
    for i, d in enumerate(mats):
        _need(d["packed"], torch.uint8, 2, f"matrix {i} packed")
        N = d["packed"].shape[0]
        if d["packed"].shape[1] * 4 != K:
            raise ValueError(f"matrix {i}: packed has {d['packed'].shape[1]} bytes per row, expected K/4 = {K // 4}")
        _shape(d["w_scale"], torch.float32, (1,), f"matrix {i} w_scale")
        for key in ("residual", "mul_by", "y_out"):
            _shape(d.get(key), torch.float32, (M, N), f"matrix {i} {key}")
        if d.get("subln"):
            _shape(d.get("norm_gain"), torch.float32, (N,), f"matrix {i} norm_gain")
        _on_gpu(d["packed"], d["w_scale"], d.get("residual"), d.get("mul_by"), d.get("y_out"), d.get("norm_gain"))
    arr = (Group * len(mats))()
    results = []
    for i, d in enumerate(mats):
        N = d["packed"].shape[0]
        res = {}
        g = arr[i]
        g.packed, g.w_scale, g.N = d["packed"].data_ptr(), d["w_scale"].data_ptr(), N
        flags = BL_EPI_RELU2 if d.get("relu2") else 0
        if d.get("residual") is not None:
            flags |= BL_EPI_RESIDUAL
            g.epi.residual = d["residual"].data_ptr()
        if d.get("mul_by") is not None:
            flags |= BL_EPI_MUL
            g.epi.mul_by = d["mul_by"].data_ptr()
        if d.get("subln"):
            flags |= BL_EPI_SUBLN_QUANT
            res["q"] = torch.empty((M, N), dtype=torch.int8, device=dev)
            res["q_scale"] = torch.empty(M, dtype=torch.float32, device=dev)
            res["q_rowsum"] = torch.empty(M, dtype=torch.int32, device=dev)
            g.epi.out_q, g.epi.out_q_scale = res["q"].data_ptr(), res["q_scale"].data_ptr()
            g.epi.out_q_rowsum = res["q_rowsum"].data_ptr()
            g.epi.norm_gain = None if d.get("norm_gain") is None else d["norm_gain"].data_ptr()
            g.epi.norm_eps = float(d.get("eps", RMS_EPS))
        g.epi.flags = flags
        y = d.get("y_out")
        if y is None:
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
        res["y"] = y
        g.Y = y.data_ptr()
        if d.get("want_acc"):
            res["acc"] = torch.empty((M, N), dtype=torch.int32, device=dev)
            g.acc_out = res["acc"].data_ptr()
        results.append(res)
    return arr, results


def forward_grouped(xq: torch.Tensor, x_scale: torch.Tensor, x_rowsum: torch.Tensor, mats: Sequence[dict]):
    """Several BitLinears of the same K on the same int8 rows in one call
    (bitlinear_forward_grouped).  Each dict of ``mats`` holds ``packed``,
    ``w_scale`` and optionally ``relu2``, ``residual``, ``mul_by``, ``subln``,
    ``norm_gain``, ``eps``, ``want_acc``, ``y_out``; returns one result dict
    per matrix, as :func:`forward` does."""
    lib = load()
    _need(xq, torch.int8, 2, "xq")
    M, K = xq.shape
    _shape(x_scale, torch.float32, (M,), "x_scale")
    _shape(x_rowsum, torch.int32, (M,), "x_rowsum")
    _on_gpu(xq, x_scale, x_rowsum)
    arr, results = _groups(mats, M, K, xq.device)
    _check(lib.bitlinear_forward_grouped(_p(xq), _p(x_scale), _p(x_rowsum), M, K, arr, len(mats), _stream(xq.device)))
    return results


def quant_forward_grouped(X: torch.Tensor, mats: Sequence[dict], rmsnorm: bool = False,
                          norm_gain: Optional[torch.Tensor] = None, eps: float = RMS_EPS,
                          ws: Optional[torch.Tensor] = None):
    """bitlinear_quant_forward_grouped: quantise fp32 rows X (optional
    RMSNorm) and apply every matrix of ``mats`` (as in
    :func:`forward_grouped`) to them; one launch for a few tokens against
    many tiles.  ``ws`` (uint8, at least the call's workspace size) may be
    passed to avoid an allocation."""
    lib = load()
    _need(X, torch.float32, 2, "X")
    M, K = X.shape
    _shape(norm_gain, torch.float32, (K,), "norm_gain")
    _on_gpu(X, norm_gain)
    arr, results = _groups(mats, M, K, X.device)
    nb = lib.bitlinear_quant_forward_grouped_workspace_bytes(M, K)
    if ws is None:
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device=X.device)
    _need(ws, torch.uint8, 1, "ws")
    if ws.numel() < nb:
        raise ValueError(f"ws holds {ws.numel()} bytes, the call needs {nb}")
    _on_gpu(ws)
    _check(lib.bitlinear_quant_forward_grouped(_p(X), M, K, BL_QUANT_RMSNORM if rmsnorm else 0, _p(norm_gain),
                                               float(eps), arr, len(mats), _p(ws), ws.numel(), _stream(X.device)))
    return results


class QuantForward:
    """Reusable launcher for bitlinear_quant_forward (fp32 rows -> int8 ->
    BitLinear -> epilogue) holding its workspace for up to ``max_m`` rows."""

    def __init__(self, packed: torch.Tensor, w_scale: torch.Tensor, max_m: int, rmsnorm: bool = False,
                 norm_gain: Optional[torch.Tensor] = None, eps: float = RMS_EPS, relu2: bool = False):
        self.lib = load()
        _need(packed, torch.uint8, 2, "packed")
        self.packed, self.w_scale = packed, w_scale
        self.N, self.K = packed.shape[0], packed.shape[1] * 4
        _shape(w_scale, torch.float32, (1,), "w_scale")
        _shape(norm_gain, torch.float32, (self.K,), "norm_gain")
        _on_gpu(packed, w_scale, norm_gain)
        self.qflags = BL_QUANT_RMSNORM if rmsnorm else 0
        self.gain, self.eps, self.relu2 = norm_gain, float(eps), relu2
        self.ws = _workspace(self.lib.bitlinear_quant_forward_workspace_bytes(max_m, self.K, self.N),
                             packed.device)

    def __call__(self, X: torch.Tensor, residual: Optional[torch.Tensor] = None,
                 y_out: Optional[torch.Tensor] = None, mul_by: Optional[torch.Tensor] = None) -> torch.Tensor:
        _need(X, torch.float32, 2, "X")
        M = X.shape[0]
        if X.shape[1] != self.K:
            raise ValueError(f"X has {X.shape[1]} columns, the weights K = {self.K}")
        for t, name in ((residual, "residual"), (mul_by, "mul_by"), (y_out, "y_out")):
            _shape(t, torch.float32, (M, self.N), name)
        _on_gpu(X, residual, mul_by, y_out)
        y = y_out if y_out is not None else torch.empty((M, self.N), dtype=torch.float32, device=X.device)
        epi = Epilogue()
        epi.flags = ((BL_EPI_RELU2 if self.relu2 else 0) | (BL_EPI_RESIDUAL if residual is not None else 0)
                     | (BL_EPI_MUL if mul_by is not None else 0))
        if residual is not None:
            epi.residual = residual.data_ptr()
        if mul_by is not None:
            epi.mul_by = mul_by.data_ptr()
        _check(self.lib.bitlinear_quant_forward(_p(X), M, self.K, self.qflags, _p(self.gain), self.eps,
                                                _p(self.packed), _p(self.w_scale), self.N, ctypes.byref(epi),
                                                _p(y), _p(self.ws), 0 if self.ws is None else self.ws.numel(),
                                                _stream(X.device)))
        return y


def quant_forward(X: torch.Tensor, packed: torch.Tensor, w_scale: torch.Tensor, rmsnorm: bool = False,
                  norm_gain: Optional[torch.Tensor] = None, eps: float = RMS_EPS, relu2: bool = False,
                  residual: Optional[torch.Tensor] = None, y_out: Optional[torch.Tensor] = None,
                  mul_by: Optional[torch.Tensor] = None):
    """Quantise fp32 X [M][K] and apply the BitLinear in one call; returns Y [M][N]."""
    return QuantForward(packed, w_scale, X.shape[0], rmsnorm, norm_gain, eps, relu2)(X, residual, y_out, mul_by)


def latent_forward(X: torch.Tensor, W: torch.Tensor, rmsnorm: bool = False,
                   norm_gain: Optional[torch.Tensor] = None, eps: float = RMS_EPS, relu2: bool = False,
                   residual: Optional[torch.Tensor] = None, mul_by: Optional[torch.Tensor] = None,
                   y_out: Optional[torch.Tensor] = None, w_scale_out: Optional[torch.Tensor] = None):
    """BitLinear from latent fp32 or bf16 weights W [N][K] (ternarised inside
    the call) on fp32 X [M][K]; returns Y [M][N] (the fake-quant forward)."""
    lib = load()
    _need(X, torch.float32, 2, "X")
    if W.dtype not in (torch.float32, torch.bfloat16) or W.dim() != 2 or not W.is_contiguous():
        raise ValueError("W must be a contiguous 2-D float32 or bfloat16 tensor")
    M, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError(f"W has {W.shape[1]} columns, X has K = {K}")
    for t, name in ((residual, "residual"), (mul_by, "mul_by"), (y_out, "y_out")):
        _shape(t, torch.float32, (M, N), name)
    _shape(norm_gain, torch.float32, (K,), "norm_gain")
    _shape(w_scale_out, torch.float32, (1,), "w_scale_out")
    _on_gpu(X, W, residual, mul_by, y_out, norm_gain, w_scale_out)
    dev = X.device
    y = y_out if y_out is not None else torch.empty((M, N), dtype=torch.float32, device=dev)
    epi = Epilogue()
    epi.flags = ((BL_EPI_RELU2 if relu2 else 0) | (BL_EPI_RESIDUAL if residual is not None else 0)
                 | (BL_EPI_MUL if mul_by is not None else 0))
    if residual is not None:
        epi.residual = residual.data_ptr()
    if mul_by is not None:
        epi.mul_by = mul_by.data_ptr()
    ws = _workspace(lib.bitlinear_latent_forward_workspace_bytes(M, K, N), dev)
    dt = BL_DTYPE_BF16 if W.dtype == torch.bfloat16 else BL_DTYPE_F32
    _check(lib.bitlinear_latent_forward(_p(X), M, K, BL_QUANT_RMSNORM if rmsnorm else 0, _p(norm_gain), float(eps),
                                        _p(W), dt, N, ctypes.byref(epi), _p(y), _p(w_scale_out), _p(ws),
                                        0 if ws is None else ws.numel(), _stream(dev)))
    return y


def make_layers(layers: Sequence[dict], H: Optional[int] = None, F: Optional[int] = None):
    """Host array of FFN layer descriptors from dicts of device tensors
    (keys: up, up_scale, down, down_scale, optional gate, gate_scale, pre_norm_gain,
    sub_norm_gain); with H and F, every tensor's shape is checked."""
    arr = (FFNLayer * len(layers))()
    for i, L in enumerate(layers):
        if H is not None and F is not None:
            _shape(L["up"], torch.uint8, (F, H // 4), f"layer {i} up")
            _shape(L["down"], torch.uint8, (H, F // 4), f"layer {i} down")
            _shape(L.get("gate"), torch.uint8, (F, H // 4), f"layer {i} gate")
            for k in ("up_scale", "down_scale", "gate_scale"):
                _shape(L.get(k), torch.float32, (1,), f"layer {i} {k}")
            _shape(L.get("pre_norm_gain"), torch.float32, (H,), f"layer {i} pre_norm_gain")
            _shape(L.get("sub_norm_gain"), torch.float32, (F,), f"layer {i} sub_norm_gain")
            _on_gpu(*(L.get(k) for k in ("up", "down", "gate", "up_scale", "down_scale", "gate_scale",
                                         "pre_norm_gain", "sub_norm_gain")))
        arr[i].pre_norm_gain = None if L.get("pre_norm_gain") is None else L["pre_norm_gain"].data_ptr()
        arr[i].up = L["up"].data_ptr()
        arr[i].up_scale = L["up_scale"].data_ptr()
        arr[i].gate = None if L.get("gate") is None else L["gate"].data_ptr()
        arr[i].gate_scale = None if L.get("gate_scale") is None else L["gate_scale"].data_ptr()
        arr[i].sub_norm_gain = None if L.get("sub_norm_gain") is None else L["sub_norm_gain"].data_ptr()
        arr[i].down = L["down"].data_ptr()
        arr[i].down_scale = L["down_scale"].data_ptr()
    return arr


class FFNStack:
    """Reusable launcher for bitnet_ffn_forward: holds the layer descriptors
    and a workspace sized for up to ``max_m`` tokens."""

    def __init__(self, layers: Sequence[dict], H: int, F: int, max_m: int, device,
                 pre_norm: bool = True, residual: bool = True, eps: float = RMS_EPS, persistent: bool = False):
        self.lib = load()
        self._keep = list(layers)
        self.arr = make_layers(layers, H, F)
        self.n = len(layers)
        self.H, self.F = H, F
        self.flags = ((BL_FFN_PRE_NORM if pre_norm else 0) | (BL_FFN_RESIDUAL if residual else 0)
                      | (BL_FFN_PERSISTENT if persistent else 0))
        self.eps = float(eps)
        self.ws = _workspace(self.lib.bitnet_ffn_workspace_bytes(max_m, H, F), device)

    def __call__(self, hidden: torch.Tensor) -> torch.Tensor:
        _need(hidden, torch.float32, 2, "hidden")
        M = hidden.shape[0]
        if hidden.shape[1] != self.H:
            raise ValueError(f"hidden has {hidden.shape[1]} columns, the stack's H = {self.H}")
        _on_gpu(hidden)
        _check(self.lib.bitnet_ffn_forward(self.arr, self.n, _p(hidden), M, self.H, self.F, self.flags,
                                           self.eps, _p(self.ws), 0 if self.ws is None else self.ws.numel(),
                                           _stream(hidden.device)))
        return hidden


def ffn_forward_noalloc(layers: Sequence[dict], hidden: torch.Tensor, pre_norm: bool = True,
                        residual: bool = True, eps: float = RMS_EPS) -> torch.Tensor:
    """The FFN stack in place on hidden [M][H] with the library's fixed
    scratch (bitnet_ffn_forward_noalloc: no workspace, nothing allocated
    beyond the layer descriptors' host array)."""
    lib = load()
    _need(hidden, torch.float32, 2, "hidden")
    M, H = hidden.shape
    F = layers[0]["up"].shape[0] if layers else 64
    arr = make_layers(layers, H, F)
    _on_gpu(hidden)
    flags = (BL_FFN_PRE_NORM if pre_norm else 0) | (BL_FFN_RESIDUAL if residual else 0)
    _check(lib.bitnet_ffn_forward_noalloc(arr, len(layers), _p(hidden), M, H, F, flags, float(eps),
                                          _stream(hidden.device)))
    return hidden


def ffn_forward(layers: Sequence[dict], hidden: torch.Tensor, pre_norm: bool = True,
                residual: bool = True, eps: float = RMS_EPS) -> torch.Tensor:
    """Run the FFN stack in place on hidden [M][H]; returns hidden."""
    M, H = hidden.shape
    F = layers[0]["up"].shape[0] if layers else 64
    return FFNStack(layers, H, F, max(M, 1), hidden.device, pre_norm, residual, eps)(hidden)
