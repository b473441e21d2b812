"""bitnet_ffn_forward_noalloc, the FFN stack for callers that cannot
allocate (its scratch is the library's fixed device array), against
bitnet_ffn_forward with a caller workspace, through the C ABI: bit-identical
hidden states on calls in a row with fewer tokens each time (GEMM, batched and
decode paths, plain and gated layers), and too many tokens rejected before
anything runs."""
import ctypes

import numpy as np
import pytest

from bit_gemm_absmax_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from bit_gemm_absmax_amd import bitlinear as bl  # noqa: E402

DEV = torch.device("cuda:0")
H, F = synth.HIDDEN, synth.FFN
FLAGS = bl.BL_FFN_PRE_NORM | bl.BL_FFN_RESIDUAL


def gpu_layers(rng, n, gated):
    out = []
    for _ in range(n):
        L = {}
        names = (("gate", F, H),) if gated else ()
        for name, rows, cols in names + (("up", F, H), ("down", H, F)):
            p, s = bl.pack_weights(torch.from_numpy(synth.weights(rng, rows, cols)).to(DEV))
            L[name], L[name + "_scale"] = p, s
        L["pre_norm_gain"] = torch.from_numpy(synth.gains(rng, H)).to(DEV)
        L["sub_norm_gain"] = torch.from_numpy(synth.gains(rng, F)).to(DEV)
        out.append(L)
    return out


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def with_workspace(lib, arr, n, h, flags=FLAGS):
    M = h.shape[0]
    nb = lib.bitnet_ffn_workspace_bytes(M, H, F)
    ws = torch.empty(nb, dtype=torch.uint8, device=DEV)
    rc = lib.bitnet_ffn_forward(arr, n, ctypes.c_void_p(h.data_ptr()), M, H, F, flags, 1e-5,
                                ctypes.c_void_p(ws.data_ptr()), nb, stream())
    assert rc == bl.BL_OK, lib.bitlinear_last_error()
    torch.cuda.synchronize()
    del ws


def no_alloc(lib, arr, n, h, flags=FLAGS):
    M = h.shape[0]
    rc = lib.bitnet_ffn_forward_noalloc(arr, n, ctypes.c_void_p(h.data_ptr()), M, H, F, flags, 1e-5, stream())
    assert rc == bl.BL_OK, lib.bitlinear_last_error()
    torch.cuda.synchronize()


@pytest.mark.parametrize("gated", [False, True])
def test_noalloc_equals_workspace_entry(gated):
    lib = bl.load()
    rng = np.random.default_rng(8100 + gated)
    layers = gpu_layers(rng, 2, gated)
    arr = bl.make_layers(layers, H, F)
    for M in (300, 40, 3, 1):   # each call after a larger one: the scratch holds the last call's data
        print(f"[no-alloc] gated={gated} M={M}", flush=True)
        h0 = torch.from_numpy(synth.activations(rng, M, H, outliers=True)).to(DEV)
        a, b = h0.clone(), h0.clone()
        with_workspace(lib, arr, len(layers), a)
        no_alloc(lib, arr, len(layers), b)
        assert torch.equal(a, b), f"M={M}: no-alloc entry differs from the workspace entry"
        assert not torch.equal(b, h0)


def test_noalloc_persistent_equals_workspace_entry():
    """With BL_FFN_PERSISTENT (one token, every layer in one launch, its
    descriptors and ready flags in the scratch): the no-alloc entry gives the
    workspace entry's hidden state on two calls in a row."""
    lib = bl.load()
    rng = np.random.default_rng(8300)
    layers = gpu_layers(rng, 3, False)
    arr = bl.make_layers(layers, H, F)
    flags = FLAGS | bl.BL_FFN_PERSISTENT
    for rep in range(2):
        print(f"[no-alloc] persistent call {rep}", flush=True)
        h0 = torch.from_numpy(synth.activations(rng, 1, H, outliers=True)).to(DEV)
        a, b = h0.clone(), h0.clone()
        with_workspace(lib, arr, len(layers), a, flags)
        no_alloc(lib, arr, len(layers), b, flags)
        assert torch.equal(a, b), f"call {rep}: persistent no-alloc entry differs from the workspace entry"
        assert not torch.equal(b, h0)


def test_noalloc_rejects_beyond_its_scratch():
    lib = bl.load()
    rng = np.random.default_rng(8200)
    layers = gpu_layers(rng, 1, False)
    arr = bl.make_layers(layers, H, F)
    top = max(m for m in range(1700, 1900) if lib.bitnet_ffn_workspace_bytes(m, H, F) <= bl.NOALLOC_MAX_BYTES)
    assert top >= 1800
    M = top + 1
    assert lib.bitnet_ffn_workspace_bytes(M, H, F) > bl.NOALLOC_MAX_BYTES
    h = torch.from_numpy(synth.activations(rng, M, H)).to(DEV)
    before = h.clone()
    rc = lib.bitnet_ffn_forward_noalloc(arr, 1, ctypes.c_void_p(h.data_ptr()), M, H, F, FLAGS, 1e-5, stream())
    assert rc == bl.BL_ERR_WORKSPACE
    assert b"scratch" in lib.bitlinear_last_error()
    torch.cuda.synchronize()
    assert torch.equal(h, before)
    # and the entry point still works after the rejection
    h2 = torch.from_numpy(synth.activations(rng, 2, H)).to(DEV)
    a, b = h2.clone(), h2.clone()
    with_workspace(lib, arr, 1, a)
    no_alloc(lib, arr, 1, b)
    assert torch.equal(a, b)
