"""Comparison rules between the HIP path and the CPU oracle.

R1  packed bytes, scales, int8 activations, row sums and int32 accumulators
    must be bit-identical.
R2  fp32 outputs: |g - o| <= 1e-5 * max(|o|, 1e-6 * max_row |o|) elementwise.
R3  a requantised int8 value computed from fp32 data may differ by exactly 1
    only where the oracle's pre-rounding value t = z * (127 / gamma) lies
    within 1e-4 of a rounding midpoint; its scale must still match exactly.
"""
import sys

import numpy as np

import oracle

REL_TOL = 1e-5


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def assert_y_close(got, want, what="y"):
    got = np.asarray(got, np.float32)
    want = np.asarray(want, np.float32)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    row_max = np.abs(want).max(axis=-1, keepdims=True) if want.size else want
    floor = np.maximum(np.abs(want), 1e-6 * row_max)
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = err > REL_TOL * floor
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond 1e-5 rel, e.g. "
                             + ", ".join(f"{tuple(i)} got {got[tuple(i)]!r} want {want[tuple(i)]!r}" for i in idx))
    return int(np.count_nonzero(np.abs(want) < 1e-6 * row_max))


def assert_exact(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if not np.array_equal(got, want):
        idx = np.argwhere(got != want)[:5]
        raise AssertionError(f"{what}: {int((got != want).sum())} mismatches, e.g. "
                             + ", ".join(f"{tuple(i)} got {got[tuple(i)]} want {want[tuple(i)]}" for i in idx))


def check_requant(z, q_gpu, scale_gpu, rowsum_gpu=None, what="requant"):
    """Teacher-forced R3 check of an absmax quantisation of the fp32 rows z
    (the oracle's own values) against the GPU's (q, scale, rowsum).
    Returns the number of explained near-tie flips."""
    xq, g, rs = oracle.quant_act(z)
    assert_exact(scale_gpu, g, f"{what}: scale")
    q_gpu = np.asarray(q_gpu)
    diff = np.argwhere(q_gpu != xq)
    if len(diff):
        s = (np.float32(127.0) / g.astype(np.float32)).astype(np.float32)
        t = (z.astype(np.float32) * s[:, None]).astype(np.float32).astype(np.float64)
        for m, k in diff:
            assert abs(int(q_gpu[m, k]) - int(xq[m, k])) == 1, (what, m, k)
            frac = t[m, k] - np.floor(t[m, k])
            assert abs(frac - 0.5) < 1e-4, (what, m, k, t[m, k])
    if rowsum_gpu is not None:
        assert_exact(rowsum_gpu, q_gpu.astype(np.int64).sum(axis=1).astype(np.int32), f"{what}: rowsum")
    return len(diff)


def explain_gamma_mismatch(W, got):
    """gamma_w may differ only when the binary64 mean lies within N*K*2^-53
    relative of a binary32 rounding midpoint (summation order)."""
    exact = np.abs(W.astype(np.float64)).sum() / W.size
    lo = np.float32(exact)
    nxt = np.nextafter(lo, np.float32(np.inf)) if exact >= float(lo) else np.nextafter(lo, np.float32(-np.inf))
    mid = (float(lo) + float(nxt)) / 2
    return abs(exact - mid) <= W.size * 2.0 ** -53 * exact and got in (lo, nxt)
