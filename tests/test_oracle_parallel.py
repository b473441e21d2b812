"""The OpenMP build of the oracle (liboracle_mt.so) against the one-core
build (liboracle.so): the same C source, with only the outermost loop of each
step split over threads, so every result must be bit-identical.  The parity
tests at the workloads' full sizes and the benchmark's all-core CPU baseline
use the OpenMP build; these tests are what lets them stand in for the pinned
one-core oracle."""
import numpy as np
import pytest

import oracle
from bit_gemm_absmax_amd import synth


def both(fn):
    """fn() on the one-core build, then with 4 (or more) threads."""
    with oracle.parallel(1):
        a = fn()
    with oracle.parallel(max(4, oracle.default_threads())) as n:
        assert n > 1 and oracle.threads() == n
        b = fn()
    assert oracle.threads() == 1
    return a, b


def assert_same(a, b):
    if isinstance(a, dict):
        assert a.keys() == b.keys()
        for k in a:
            assert_same(a[k], b[k])
    elif isinstance(a, (tuple, list)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            assert_same(x, y)
    else:
        a, b = np.atleast_1d(np.asarray(a)), np.atleast_1d(np.asarray(b))
        assert a.dtype == b.dtype and a.shape == b.shape
        assert a.tobytes() == b.tobytes()


def test_thread_switch():
    assert oracle.threads() == 1
    with oracle.parallel(3) as n:
        assert n == 3
    assert oracle.threads() == 1
    assert oracle.set_threads(1) == 1


@pytest.mark.parametrize("M,K,N", [(1, 2560, 6912), (37, 640, 200), (130, 256, 1000)])
def test_steps_identical(M, K, N):
    rng = np.random.default_rng(M + K + N)
    W = synth.weights(rng, N, K)
    X = synth.activations(rng, M, K, outliers=True)
    G = synth.gains(rng, K)
    A = synth.activations(rng, M, N)

    def run():
        q, g = oracle.quantize_weights(W)
        r = oracle.bitlinear(X, q, g, relu_sq=True)
        z = oracle.rmsnorm(X, G)
        return {"q": q, "g": g, "xq": r["xq"], "gx": r["gamma_x"], "rs": r["rowsum"], "acc": r["acc"],
                "y": r["y"], "z": z, "zq": oracle.quant_act(z), "add": oracle.add(A, r["y"]),
                "mul": oracle.mul(r["y"], A)}

    a, b = both(run)
    assert_same(a, b)


@pytest.mark.parametrize("gated", [False, True])
def test_ffn_layer_identical(gated):
    rng = np.random.default_rng(77 + gated)
    M, Hd, F = 9, 256, 640
    qg = oracle.quantize_weights(synth.weights(rng, F, Hd))
    qu = oracle.quantize_weights(synth.weights(rng, F, Hd))
    qd = oracle.quantize_weights(synth.weights(rng, Hd, F))
    H = synth.activations(rng, M, Hd)
    pre, sub = synth.gains(rng, Hd), synth.gains(rng, F)

    def run():
        if gated:
            return oracle.ffn_layer_gated(H, qg[0], qg[1], qu[0], qu[1], qd[0], qd[1], pre_gain=pre,
                                          sub_gain=sub, intermediates=True)
        return oracle.ffn_layer(H, qu[0], qu[1], qd[0], qd[1], pre_gain=pre, sub_gain=sub,
                                intermediates=True)

    a, b = both(run)
    assert_same(a, b)
