"""Host-side checks of the C ABI: the library loads, exports every function
include/bitlinear.h declares, and rejects bad arguments before launching
anything.  No call here reaches a kernel launch, so these run without a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

from bit_gemm_absmax_amd import bitlinear as bl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?[\s\*](\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n.startswith(("bitlinear_", "bitnet_"))))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bl.LIB_PATH):
        from bit_gemm_absmax_amd import build
        build.build()
    return bl.load()


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("bitlinear_pack_weights", "bitlinear_quant_act", "bitlinear_forward", "bitnet_ffn_forward"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bl.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None
    assert set(bl.SYMBOLS) == set(declared_functions())


def test_version_and_status_strings(lib):
    assert lib.bitlinear_abi_version() == (1 << 16) | 2
    for s in range(-6, 1):
        assert lib.bitlinear_status_string(s)
    assert lib.bitlinear_status_string(-99) == b"unknown status"


def test_workspace_queries(lib):
    assert lib.bitlinear_pack_workspace_bytes(6912, 2560) >= 8 * 1024
    assert lib.bitlinear_pack_workspace_bytes(0, 64) == 0
    assert lib.bitlinear_forward_workspace_bytes(4096, 2560, 6912, 0) >= 4096 * 4
    with_y = lib.bitlinear_forward_workspace_bytes(4096, 2560, 6912, bl.BL_EPI_SUBLN_QUANT)
    assert with_y >= 4096 * 6912 * 4
    ffn = lib.bitnet_ffn_workspace_bytes(32, 2560, 6912)
    assert ffn >= 32 * 2560 + 32 * 6912 * 5
    assert lib.bitnet_ffn_workspace_bytes(0, 2560, 6912) == 0


# Fake, aligned, never-dereferenced device addresses: every call below fails
# validation (or has M == 0) before anything touches them.
A = ctypes.c_void_p(1 << 20)
B = ctypes.c_void_p(2 << 20)
C = ctypes.c_void_p(3 << 20)
D = ctypes.c_void_p(4 << 20)
MIS = ctypes.c_void_p((5 << 20) + 4)


def test_pack_validation(lib):
    f = lib.bitlinear_pack_weights
    assert f(None, 4, 64, B, C, D, 1 << 20, None) == bl.BL_ERR_NULL
    assert b"required" in lib.bitlinear_last_error()
    assert f(A, 0, 64, B, C, D, 1 << 20, None) == bl.BL_ERR_SHAPE
    assert f(A, 4, 96, B, C, D, 1 << 20, None) == bl.BL_ERR_SHAPE
    assert f(A, 4, 0, B, C, D, 1 << 20, None) == bl.BL_ERR_SHAPE
    assert f(MIS, 4, 64, B, C, D, 1 << 20, None) == bl.BL_ERR_ALIGN
    assert f(A, 4, 64, B, C, None, 0, None) == bl.BL_ERR_WORKSPACE
    assert f(A, 4, 64, B, C, D, 16, None) == bl.BL_ERR_WORKSPACE
    assert f(A, 4, 64, B, C, MIS, 1 << 20, None) == bl.BL_ERR_ALIGN


def test_quant_validation(lib):
    f = lib.bitlinear_quant_act
    assert f(None, 1, 64, 0, None, 1e-5, B, C, D, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0x8, None, 1e-5, B, C, D, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, -1, 64, 0, None, 1e-5, B, C, D, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 100, 0, None, 1e-5, B, C, D, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 65536, 0, None, 1e-5, B, C, D, None) == bl.BL_ERR_UNSUPPORTED
    assert f(MIS, 1, 64, 0, None, 1e-5, B, C, D, None) == bl.BL_ERR_ALIGN
    # empty batch: validated, nothing launched
    assert f(A, 0, 64, 0, None, 1e-5, B, C, D, None) == bl.BL_OK
    assert lib.bitlinear_last_error() == b""


def test_forward_validation(lib):
    f = lib.bitlinear_forward
    E = bl.Epilogue
    nul = ctypes.POINTER(E)()
    assert f(None, B, None, 1, 64, C, D, 8, nul, A, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, B, None, 1, 64, C, D, 8, nul, None, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, B, None, 1, 63, C, D, 8, nul, A, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, 1, 64, C, D, 0, nul, A, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, -2, 64, C, D, 8, nul, A, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, 1, 64, C, D, 8, nul, MIS, None, None, 0, None) == bl.BL_ERR_ALIGN
    # missing workspace when the row sums must be computed
    assert f(A, B, None, 1, 64, C, D, 8, nul, A, None, None, 0, None) == bl.BL_ERR_WORKSPACE
    e = E(flags=bl.BL_EPI_RESIDUAL)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_SUBLN_QUANT)
    assert f(A, B, D, 1, 64, C, D, 64, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_SUBLN_QUANT, out_q=A.value, out_q_scale=B.value)
    assert f(A, B, D, 1, 64, C, D, 72, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_SHAPE
    e = E(flags=0x40)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    # gating product: needs mul_by, 16-byte aligned, and not with the residual add
    e = E(flags=bl.BL_EPI_MUL)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL, mul_by=MIS.value)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_ALIGN
    e = E(flags=bl.BL_EPI_MUL | bl.BL_EPI_RESIDUAL, mul_by=A.value, residual=B.value)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), A, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    # empty batch with everything else valid
    assert f(A, B, D, 0, 64, C, D, 8, nul, A, None, None, 0, None) == bl.BL_OK


def test_ffn_validation(lib):
    f = lib.bitnet_ffn_forward
    L = (bl.FFNLayer * 1)()
    L[0].up, L[0].up_scale, L[0].down, L[0].down_scale = A.value, B.value, C.value, D.value
    assert f(L, 1, None, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_NULL
    assert f(None, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_NULL
    assert f(L, -1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(L, 1, A, 1, 64, 96, 3, 1e-5, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(L, 1, A, 1, 64, 64, 0x10, 1e-5, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert f(L, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_WORKSPACE
    G = (bl.FFNLayer * 1)()
    ctypes.memmove(G, L, ctypes.sizeof(L))
    G[0].gate = A.value          # a gate needs its scale
    assert f(G, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_NULL
    G[0].gate_scale = MIS.value + 2  # and both need their alignment (4 bytes for a scale)
    assert f(G, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_ALIGN
    G[0].gate_scale = B.value    # a valid gated layer then needs the workspace
    assert f(G, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_WORKSPACE
    Z = (bl.FFNLayer * 1)()
    assert f(Z, 1, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_ERR_NULL
    assert f(L, 0, A, 1, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_OK
    assert f(L, 1, A, 0, 64, 64, 3, 1e-5, None, 0, None) == bl.BL_OK


def test_binding_raises_on_bad_tensor():
    import torch
    with pytest.raises((ValueError, TypeError)):
        bl.pack_weights(torch.zeros(4, 64))  # CPU tensor: rejected before any C call


def test_quant_forward_validation(lib):
    f = lib.bitlinear_quant_forward
    E = bl.Epilogue
    nul = ctypes.POINTER(E)()
    assert f(None, 1, 64, 0, None, 1e-5, B, C, 8, nul, D, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, nul, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0x4, None, 1e-5, B, C, 8, nul, D, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_SUBLN_QUANT)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), D, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_RESIDUAL)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), D, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), D, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL | bl.BL_EPI_RESIDUAL, mul_by=A.value, residual=B.value)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), D, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, 1, 96, 0, None, 1e-5, B, C, 8, nul, D, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 0, nul, D, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, nul, MIS, None, 0, None) == bl.BL_ERR_ALIGN
    assert f(A, 0, 64, 0, None, 1e-5, B, C, 8, nul, D, None, 0, None) == bl.BL_OK
    assert lib.bitlinear_quant_forward_workspace_bytes(64, 2560, 6912) >= 64 * 2560


def test_latent_forward_validation(lib):
    f = lib.bitlinear_latent_forward
    nul = ctypes.POINTER(bl.Epilogue)()
    F32, BF16 = bl.BL_DTYPE_F32, bl.BL_DTYPE_BF16
    assert f(A, 1, 64, 0, None, 1e-5, None, F32, 8, nul, D, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(None, 1, 64, 0, None, 1e-5, B, F32, 8, nul, D, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0, None, 1e-5, B, 7, 8, nul, D, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, 1, 96, 0, None, 1e-5, B, BF16, 8, nul, D, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 64, 0, None, 1e-5, MIS, F32, 8, nul, D, None, None, 0, None) == bl.BL_ERR_ALIGN
    assert f(A, 1, 64, 0, None, 1e-5, B, F32, 8, nul, D, None, None, 0, None) == bl.BL_ERR_WORKSPACE
    assert f(A, 0, 64, 0, None, 1e-5, B, F32, 8, nul, D, None, None, 0, None) == bl.BL_OK
    need = lib.bitlinear_latent_forward_workspace_bytes(4096, 2560, 6912)
    assert need >= 6912 * 2560 // 4 + 4096 * 2560
    assert lib.bitlinear_latent_forward_workspace_bytes(0, 2560, 6912) == 0


def test_bench_library_exports_stream_read():
    """The benchmark's read-bandwidth kernel library: built beside the main
    one, exports its one call, and rejects sizes before launching anything."""
    from bit_gemm_absmax_amd import build
    if not os.path.exists(build.BENCH_LIB):
        build.build()
    blib = ctypes.CDLL(build.BENCH_LIB)
    f = blib.blbench_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    assert f(None, 3, None, None) == -2
    assert f(None, (256 << 20) + 64, None, None) == -2
    assert f(None, 4 << 30, None, None) == -2


def _device_visible() -> bool:
    try:
        import torch
        return torch.cuda.device_count() > 0  # counting does not initialise a device
    except Exception:  # pragma: no cover
        return False


def test_no_device_gives_hip_status(lib):
    """Valid arguments with no GPU present: every compute call passes
    validation, its launch fails, and it returns BL_ERR_HIP with a message
    instead of aborting.  Runs only where no device is visible (the fake
    pointers below would otherwise reach a kernel)."""
    if _device_visible():
        pytest.skip("a GPU is visible: this test is for a host without one")
    E = bl.Epilogue
    nul = ctypes.POINTER(E)()
    WS, WSN = C, 1 << 30
    calls = {
        "pack": lambda: lib.bitlinear_pack_weights(A, 4, 64, B, D, WS, WSN, None),
        "quant": lambda: lib.bitlinear_quant_act(A, 2, 64, 0, None, 1e-5, B, D, None, None),
        "forward": lambda: lib.bitlinear_forward(A, B, None, 2, 64, D, B, 8, nul, A, None, WS, WSN, None),
        "quant_forward": lambda: lib.bitlinear_quant_forward(A, 2, 64, 0, None, 1e-5, B, D, 8, nul, A, WS, WSN, None),
        "latent_forward": lambda: lib.bitlinear_latent_forward(A, 2, 64, 0, None, 1e-5, B, bl.BL_DTYPE_F32, 8, nul,
                                                               D, None, WS, WSN, None),
    }
    for name, call in calls.items():
        assert call() == bl.BL_ERR_HIP, name
        assert lib.bitlinear_last_error(), name
    layer = bl.FFNLayer(up=A.value, up_scale=B.value, down=D.value, down_scale=B.value)
    arr = (bl.FFNLayer * 1)(layer)
    assert lib.bitnet_ffn_forward(arr, 1, A, 2, 64, 64, 0, 1e-5, WS, WSN, None) == bl.BL_ERR_HIP
