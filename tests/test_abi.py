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
    assert lib.bitlinear_abi_version() == (1 << 16) | 4
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
Y = ctypes.c_void_p(6 << 20)   # an output far from every input above


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
    assert f(None, B, None, 1, 64, C, D, 8, nul, Y, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, B, None, 1, 64, C, D, 8, nul, None, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, B, None, 1, 63, C, D, 8, nul, Y, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, 1, 64, C, D, 0, nul, Y, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, -2, 64, C, D, 8, nul, Y, None, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, B, None, 1, 64, C, D, 8, nul, MIS, None, None, 0, None) == bl.BL_ERR_ALIGN
    # missing workspace when the row sums must be computed
    assert f(A, B, None, 1, 64, C, D, 8, nul, Y, None, None, 0, None) == bl.BL_ERR_WORKSPACE
    e = E(flags=bl.BL_EPI_RESIDUAL)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_SUBLN_QUANT)
    assert f(A, B, D, 1, 64, C, D, 64, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_SUBLN_QUANT, out_q=A.value, out_q_scale=B.value)
    assert f(A, B, D, 1, 64, C, D, 72, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_SHAPE
    e = E(flags=0x40)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    # gating product: needs mul_by, 16-byte aligned, and not with the residual add
    e = E(flags=bl.BL_EPI_MUL)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL, mul_by=MIS.value)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_ALIGN
    e = E(flags=bl.BL_EPI_MUL | bl.BL_EPI_RESIDUAL, mul_by=A.value, residual=B.value)
    assert f(A, B, D, 1, 64, C, D, 8, ctypes.byref(e), Y, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    # empty batch with everything else valid
    assert f(A, B, D, 0, 64, C, D, 8, nul, Y, None, None, 0, None) == bl.BL_OK


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


def test_ffn_noalloc_validation(lib):
    """The no-allocation FFN entry point checks its arguments as the
    workspace one does, and refuses shapes whose scratch exceeds its fixed
    array (64 MiB: about 1800 tokens at hidden 2560 / intermediate 6912) before any
    device call."""
    f = lib.bitnet_ffn_forward_noalloc
    L = (bl.FFNLayer * 1)()
    L[0].up, L[0].up_scale, L[0].down, L[0].down_scale = A.value, B.value, C.value, D.value
    assert f(L, 1, None, 1, 64, 64, 3, 1e-5, None) == bl.BL_ERR_NULL
    assert f(L, 1, A, 1, 64, 96, 3, 1e-5, None) == bl.BL_ERR_SHAPE
    assert f(L, 1, A, 1, 64, 64, 0x10, 1e-5, None) == bl.BL_ERR_UNSUPPORTED
    assert f(L, 1, MIS, 1, 64, 64, 3, 1e-5, None) == bl.BL_ERR_ALIGN
    assert f(L, 0, A, 1, 64, 64, 3, 1e-5, None) == bl.BL_OK
    assert f(L, 1, A, 0, 64, 64, 3, 1e-5, None) == bl.BL_OK
    top = max(m for m in range(1700, 1900) if lib.bitnet_ffn_workspace_bytes(m, 2560, 6912) <= bl.NOALLOC_MAX_BYTES)
    assert top >= 1800
    assert f(L, 1, A, top + 1, 2560, 6912, 3, 1e-5, None) == bl.BL_ERR_WORKSPACE
    assert b"scratch" in lib.bitlinear_last_error()


def test_binding_raises_on_bad_tensor():
    import torch
    with pytest.raises((ValueError, TypeError)):
        bl.pack_weights(torch.zeros(4, 64))  # CPU tensor: rejected before any C call


def test_binding_checks_shapes_before_any_call():
    """Every tensor argument's dtype and exact shape is checked against M, K
    and N before the library is called (the C layer trusts the sizes); CPU
    tensors of the right shapes are then refused as not on the GPU."""
    import torch
    M, K, N = 3, 128, 40
    xq = torch.zeros(M, K, dtype=torch.int8)
    xs, rs = torch.zeros(M), torch.zeros(M, dtype=torch.int32)
    packed, ws = torch.zeros(N, K // 4, dtype=torch.uint8), torch.zeros(1)
    good = dict(x_rowsum=rs)
    cases = [
        (dict(x_scale=torch.zeros(M + 1)), "x_scale"),
        (dict(x_rowsum=torch.zeros(M, dtype=torch.int64)), "x_rowsum"),
        (dict(w_scale=torch.zeros(2)), "w_scale"),
        (dict(residual=torch.zeros(M, N + 1)), "residual"),
        (dict(mul_by=torch.zeros(M + 1, N)), "mul_by"),
        (dict(y_out=torch.zeros(M, N - 1)), "y_out"),
        (dict(subln=True, norm_gain=torch.zeros(K)), "norm_gain"),
    ]
    for kw, name in cases:
        args = dict(xq=xq, x_scale=xs, packed=packed, w_scale=ws, **good)
        args.update(kw)
        with pytest.raises((ValueError, TypeError), match=name):
            bl.forward(**args)
    with pytest.raises(ValueError, match="GPU"):
        bl.forward(xq, xs, packed, ws, x_rowsum=rs)
    with pytest.raises(ValueError, match="bytes per row"):
        bl.forward(xq, xs, torch.zeros(N, K // 4 + 16, dtype=torch.uint8), ws)
    X = torch.zeros(M, K)
    with pytest.raises(ValueError, match="norm_gain"):
        bl.quant_act(X, rmsnorm=True, norm_gain=torch.zeros(K + 4))
    with pytest.raises(ValueError, match="Xq"):
        bl.quant_act(X, out=(torch.zeros(M, K - 64, dtype=torch.int8), xs, rs))
    with pytest.raises(ValueError, match="GPU"):
        bl.quant_act(X)
    with pytest.raises(ValueError, match="columns"):
        bl.latent_forward(X, torch.zeros(N, K + 64))
    with pytest.raises(ValueError, match="w_scale_out"):
        bl.latent_forward(X, torch.zeros(N, K), w_scale_out=torch.zeros(2))
    with pytest.raises(ValueError, match="GPU"):
        bl.unpack_weights(packed)
    with pytest.raises(TypeError):
        bl.import_canonical(torch.zeros(N, K // 4))
    # the FFN stack: every layer tensor against H and F, and hidden against H
    H, F = 64, 128
    L = {"up": torch.zeros(F, H // 4, dtype=torch.uint8), "up_scale": torch.zeros(1),
         "down": torch.zeros(H, F // 4, dtype=torch.uint8), "down_scale": torch.zeros(1)}
    for key, bad in (("up", torch.zeros(F, H // 4 + 1, dtype=torch.uint8)), ("down_scale", torch.zeros(3)),
                     ("sub_norm_gain", torch.zeros(H)), ("gate", torch.zeros(H, F // 4, dtype=torch.uint8))):
        with pytest.raises(ValueError, match=key):
            bl.make_layers([dict(L, **{key: bad})], H, F)
    with pytest.raises(ValueError, match="GPU"):
        bl.make_layers([L], H, F)


def test_layout_validation(lib):
    for f, in_al, out_al in ((lib.bitlinear_import_canonical, 4, 16), (lib.bitlinear_export_canonical, 16, 4),
                             (lib.bitlinear_unpack_weights, 16, 16)):
        assert f(None, 4, 64, B, None) == bl.BL_ERR_NULL
        assert f(A, 4, 64, None, None) == bl.BL_ERR_NULL
        assert f(A, 0, 64, B, None) == bl.BL_ERR_SHAPE
        assert f(A, 4, 96, B, None) == bl.BL_ERR_SHAPE
        assert f(A, 4, 0, B, None) == bl.BL_ERR_SHAPE
        assert f(ctypes.c_void_p(A.value + in_al // 2), 4, 64, B, None) == bl.BL_ERR_ALIGN
        assert f(A, 4, 64, ctypes.c_void_p(B.value + out_al // 2), None) == bl.BL_ERR_ALIGN
        # input and output ranges overlap (4 x 64 weights: 64 packed bytes)
        assert f(A, 4, 64, ctypes.c_void_p(A.value + 32), None) == bl.BL_ERR_UNSUPPORTED
        assert b"overlap" in lib.bitlinear_last_error()


def test_overlap_rules(lib):
    """Outputs may not overlap inputs (or other outputs); the one allowed
    alias is Y equal to residual / mul_by.  Rejected before any launch."""
    E = bl.Epilogue
    nul = ctypes.POINTER(E)()
    M, K, N = 2, 64, 16
    # quant_forward: Y over X (in-place hidden = hidden + W.norm(hidden) with K == N)
    qf = lib.bitlinear_quant_forward
    assert qf(A, M, K, 0, None, 1e-5, B, C, K, nul, A, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert b"overlaps X" in lib.bitlinear_last_error()
    assert qf(A, M, K, 0, None, 1e-5, B, C, N, nul, ctypes.c_void_p(A.value + 256), None, 0, None) == \
        bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_RESIDUAL, residual=Y.value + 64)   # partly over Y
    assert qf(A, M, K, 0, None, 1e-5, B, C, N, ctypes.byref(e), Y, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_RESIDUAL, residual=Y.value)        # exactly Y: in place, allowed
    assert qf(A, 0, K, 0, None, 1e-5, B, C, N, ctypes.byref(e), Y, None, 0, None) == bl.BL_OK
    g = ctypes.c_void_p(Y.value + 32)                        # the gain inside Y
    assert qf(A, M, K, 1, g, 1e-5, B, C, N, nul, Y, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    lf = lib.bitlinear_latent_forward
    assert lf(A, M, K, 0, None, 1e-5, B, bl.BL_DTYPE_F32, K, nul, A, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    # forward: Y over Xq, acc over Y, out_q over the weights
    fw = lib.bitlinear_forward
    assert fw(A, B, C, M, K, D, B, N, nul, A, None, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert fw(A, B, C, M, K, D, ctypes.c_void_p(B.value + 64), N, nul, Y, Y, None, 0, None) == \
        bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_SUBLN_QUANT, out_q=D.value, out_q_scale=Y.value + 4096)
    assert fw(A, B, C, M, K, D, ctypes.c_void_p(B.value + 64), 64, ctypes.byref(e), Y, None, None, 0, None) == \
        bl.BL_ERR_UNSUPPORTED
    # quant_act: Xq over X
    qa = lib.bitlinear_quant_act
    assert qa(A, M, K, 0, None, 1e-5, ctypes.c_void_p(A.value + 128), B, C, None) == bl.BL_ERR_UNSUPPORTED
    assert qa(A, M, K, 0, None, 1e-5, B, C, C, None) == bl.BL_ERR_UNSUPPORTED   # scale over rowsum
    # ffn: hidden inside the workspace
    f = lib.bitnet_ffn_forward
    L = (bl.FFNLayer * 1)()
    L[0].up, L[0].up_scale, L[0].down, L[0].down_scale = A.value, B.value, C.value, D.value
    assert f(L, 1, ctypes.c_void_p(Y.value + 512), 1, 64, 64, 3, 1e-5, Y, 1 << 20, None) == bl.BL_ERR_UNSUPPORTED


def test_quant_forward_validation(lib):
    f = lib.bitlinear_quant_forward
    E = bl.Epilogue
    nul = ctypes.POINTER(E)()
    assert f(None, 1, 64, 0, None, 1e-5, B, C, 8, nul, Y, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, nul, None, None, 0, None) == bl.BL_ERR_NULL
    assert f(A, 1, 64, 0x4, None, 1e-5, B, C, 8, nul, Y, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_SUBLN_QUANT)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), Y, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    e = E(flags=bl.BL_EPI_RESIDUAL)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), Y, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), Y, None, 0, None) == bl.BL_ERR_NULL
    e = E(flags=bl.BL_EPI_MUL | bl.BL_EPI_RESIDUAL, mul_by=A.value, residual=B.value)
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, ctypes.byref(e), Y, None, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, 1, 96, 0, None, 1e-5, B, C, 8, nul, Y, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 0, nul, Y, None, 0, None) == bl.BL_ERR_SHAPE
    assert f(A, 1, 64, 0, None, 1e-5, B, C, 8, nul, MIS, None, 0, None) == bl.BL_ERR_ALIGN
    assert f(A, 0, 64, 0, None, 1e-5, B, C, 8, nul, Y, None, 0, None) == bl.BL_OK
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
        "forward": lambda: lib.bitlinear_forward(A, B, None, 2, 64, D, B, 8, nul, Y, None, WS, WSN, None),
        "quant_forward": lambda: lib.bitlinear_quant_forward(A, 2, 64, 0, None, 1e-5, B, D, 8, nul, Y, WS, WSN, None),
        "import": lambda: lib.bitlinear_import_canonical(A, 4, 64, B, None),
        "export": lambda: lib.bitlinear_export_canonical(A, 4, 64, B, None),
        "unpack": lambda: lib.bitlinear_unpack_weights(A, 4, 64, B, None),
        "grouped": lambda: lib.bitlinear_forward_grouped(A, B, D, 2, 64, (bl.Group * 1)(bl.Group(
            packed=C.value, w_scale=B.value, N=8, Y=Y.value)), 1, None),
        "quant_grouped": lambda: lib.bitlinear_quant_forward_grouped(A, 2, 64, 0, None, 1e-5, (bl.Group * 1)(bl.Group(
            packed=C.value, w_scale=B.value, N=8, Y=Y.value)), 1, WS, WSN, None),
        "latent_forward": lambda: lib.bitlinear_latent_forward(A, 2, 64, 0, None, 1e-5, B, bl.BL_DTYPE_F32, 8, nul,
                                                               D, None, WS, WSN, None),
    }
    for name, call in calls.items():
        assert call() == bl.BL_ERR_HIP, name
        assert lib.bitlinear_last_error(), name
    layer = bl.FFNLayer(up=A.value, up_scale=B.value, down=D.value, down_scale=B.value)
    arr = (bl.FFNLayer * 1)(layer)
    assert lib.bitnet_ffn_forward(arr, 1, A, 2, 64, 64, 0, 1e-5, WS, WSN, None) == bl.BL_ERR_HIP
    # the no-allocation entry: its scratch lookup needs a device
    assert lib.bitnet_ffn_forward_noalloc(arr, 1, A, 2, 64, 64, 0, 1e-5, None) == bl.BL_ERR_HIP
    assert lib.bitlinear_last_error()


def test_forward_grouped_validation(lib):
    """The grouped forward: group count, required row sums and outputs, each
    matrix's own checks, and no output of one matrix over another's data;
    all before any launch."""
    f = lib.bitlinear_forward_grouped
    G = (bl.Group * 5)()
    for i in range(5):
        G[i].packed, G[i].w_scale, G[i].N = C.value + i * 4096, D.value + 16 * i, 16
        G[i].Y = Y.value + i * 4096
    assert f(A, B, D, 2, 64, G, 0, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, B, D, 2, 64, G, 5, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, B, D, 2, 64, None, 2, None) == bl.BL_ERR_NULL
    assert f(A, B, None, 2, 64, G, 2, None) == bl.BL_ERR_NULL            # row sums required
    H = (bl.Group * 2)()
    ctypes.memmove(H, G, ctypes.sizeof(H))
    H[1].Y = None
    assert f(A, B, D, 2, 64, H, 2, None) == bl.BL_ERR_NULL               # Y required
    assert b"matrix 1" in lib.bitlinear_last_error()
    H[1].Y, H[1].N = Y.value + 4096, 0
    assert f(A, B, D, 2, 64, H, 2, None) == bl.BL_ERR_SHAPE
    H[1].N = 16
    H[1].Y = Y.value + 64                                                 # over matrix 0's Y
    assert f(A, B, D, 2, 64, H, 2, None) == bl.BL_ERR_UNSUPPORTED
    H[1].Y = C.value                                                      # over matrix 0's weights
    assert f(A, B, D, 2, 64, H, 2, None) == bl.BL_ERR_UNSUPPORTED
    H[1].Y = Y.value + 4096
    H[0].epi.flags, H[0].epi.residual = bl.BL_EPI_RESIDUAL, H[1].Y          # residual = matrix 1's output
    assert f(A, B, D, 2, 64, H, 2, None) == bl.BL_ERR_UNSUPPORTED
    H[0].epi.residual = H[0].Y                                            # its own Y: in place, allowed
    assert f(A, B, D, 0, 64, H, 2, None) == bl.BL_OK


def test_quant_forward_grouped_validation(lib):
    """The grouped fused quantise + forward: its own checks of X, the flags,
    K and the workspace, every check of the grouped forward against the
    workspace rows, and no output over X, the gain or the workspace; all
    before any launch."""
    f = lib.bitlinear_quant_forward_grouped
    nb = lib.bitlinear_quant_forward_grouped_workspace_bytes(2, 64)
    assert nb >= 2 * 64 + 8
    assert lib.bitlinear_quant_forward_grouped_workspace_bytes(0, 64) == 0
    WS = ctypes.c_void_p(C.value + (1 << 16))
    G = (bl.Group * 2)()
    for i in range(2):
        G[i].packed, G[i].w_scale, G[i].N = C.value + i * 4096, D.value + 16 * i, 16
        G[i].Y = Y.value + i * 4096
    assert f(None, 2, 64, 0, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_NULL
    assert f(A, 2, 64, 0x8, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    assert f(A, 2, 96, 0, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_SHAPE
    assert f(A, -1, 64, 0, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_SHAPE
    assert f(ctypes.c_void_p(A.value + 4), 2, 64, 0, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_ALIGN
    assert f(A, 2, 64, 0, None, 1e-5, G, 2, WS, nb - 1, None) == bl.BL_ERR_WORKSPACE
    assert f(A, 2, 64, 0, None, 1e-5, G, 2, None, nb, None) == bl.BL_ERR_WORKSPACE
    assert f(A, 2, 64, 0, None, 1e-5, G, 0, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    H = (bl.Group * 2)()
    ctypes.memmove(H, G, ctypes.sizeof(H))
    H[1].Y = Y.value + 64                                                  # over matrix 0's Y
    assert f(A, 2, 64, 0, None, 1e-5, H, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    H[1].Y = A.value                                                       # over X
    assert f(A, 2, 64, 0, None, 1e-5, H, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    H[1].Y = WS.value                                                      # over the workspace rows
    assert f(A, 2, 64, 0, None, 1e-5, H, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    H[1].Y = ctypes.c_void_p(B.value).value                                # over the gain
    assert f(A, 2, 64, bl.BL_QUANT_RMSNORM, B, 1e-5, H, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED
    assert f(WS, 2, 64, 0, None, 1e-5, G, 2, WS, nb, None) == bl.BL_ERR_UNSUPPORTED  # X over the workspace
    assert f(A, 0, 64, 0, None, 1e-5, G, 2, None, 0, None) == bl.BL_OK     # no rows: checks only
