"""GPU parity: every exported call of libbitlinear against the CPU oracle on
the same seeded inputs.  Small and ragged shapes are compared element by
element; the full workload shapes (hidden 2560, intermediate 6912, 30 layers,
up to 4096 tokens) run in the same launch configuration the benchmark times,
and are compared in full: the largest ones against the OpenMP build of the
oracle, which gives results identical to the one-core build (pinned by
tests/test_oracle_parallel.py)."""
import numpy as np
import pytest

import oracle
from bit_gemm_absmax_amd import synth
from tests.parity import (assert_exact, assert_y_close, check_requant, explain_gamma_mismatch, log)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from bit_gemm_absmax_amd import bitlinear as bl  # noqa: E402

DEV = torch.device("cuda:0")
oracle.set_threads(oracle.default_threads())


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def gpu_pack(W):
    p, s = bl.pack_weights(dev(W))
    return p, s


def check_pack(W, what):
    log(f"[pack] {what} N={W.shape[0]} K={W.shape[1]}")
    p, s = gpu_pack(W)
    q, g = oracle.quantize_weights(W)
    got = host(s)[0]
    if got != g:
        assert explain_gamma_mismatch(W, got), (what, got, g)
        q = oracle.ternarize(W, got)
    assert_exact(host(p), oracle.pack(q), f"{what}: packed bytes")
    return p, s, q, np.float32(got)


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("N,K", [(512, 256), (100, 192), (7, 64), (1, 64), (33, 1024)])
def test_pack_small(N, K):
    rng = np.random.default_rng(N * 7 + K)
    check_pack(synth.weights(rng, N, K), "small")


@pytest.mark.parametrize("seed", range(3))
def test_pack_rounding_boundaries(seed):
    """Entries at gamma/2 and 3 gamma/2 and up to 4 ulps either side, both
    signs, inside an N(0, 0.02) matrix: the packed codes equal the oracle's
    rint-and-clip of the binary32 quotient exactly.  gamma moves with the
    probes, so they are re-placed around the oracle's gamma until it stops
    changing."""
    rng = np.random.default_rng(5200 + seed)
    N, K = 96, 1024
    W = synth.weights(rng, N, K)
    pos = rng.choice(N * K, 72, replace=False)
    g = oracle.quantize_weights(W)[1]
    for _ in range(6):
        vals = []
        for centre in (np.float32(g) / np.float32(2), np.float32(g) * np.float32(1.5)):
            w = centre
            for _ in range(4):
                w = np.nextafter(w, np.float32(0))
            for _ in range(9):
                vals.append(w)
                w = np.nextafter(w, np.float32(np.inf))
        vals = np.array(vals + [-v for v in vals], dtype=np.float32)
        Wp = W.copy().reshape(-1)
        Wp[pos[:len(vals)]] = vals
        Wp = Wp.reshape(N, K)
        g2 = oracle.quantize_weights(Wp)[1]
        if g2 == g:
            break
        g = g2
    assert g2 == g, "probe placement did not settle"
    half = np.float32(g) / np.float32(2)
    assert half in Wp and np.nextafter(half, np.float32(np.inf)) in Wp
    check_pack(Wp, "rounding boundaries")


def test_pack_special_values():
    W = np.zeros((5, 128), np.float32)
    p, s = gpu_pack(W)
    assert host(s)[0] == np.float32(1e-5)
    assert np.all(host(p) == 0x55)
    # exact ties at W/gamma = +-0.5 and +-1.5 (gamma = 1)
    W = np.tile(np.array([1.0, -1.0, 0.5, 1.5, -0.5, 0.5, 1.5, -1.5], np.float32), (2, 8))
    check_pack(W, "ties")


@pytest.mark.parametrize("N,K", [(6912, 2560), (2560, 6912), (2560, 2560)])
def test_pack_model_shapes(N, K):
    rng = np.random.default_rng(N + K)
    check_pack(synth.weights(rng, N, K), "model")


@pytest.mark.parametrize("N,K", [(2, 64), (17, 128), (100, 192), (6912, 2560), (2560, 6912), (33, 1024)])
def test_canonical_layout_roundtrip(N, K):
    """Plain row-major 2-bit bytes (the oracle's pack_canonical) -> the tile
    layout -> back, and the tile layout -> int8: bit-exact against the
    oracle's packed bytes and q, and the GPU packer's own output exports to
    the oracle's plain bytes."""
    log(f"[layout] N={N} K={K}")
    rng = np.random.default_rng(N * 3 + K)
    W = synth.weights(rng, N, K)
    q, g = oracle.quantize_weights(W)
    canon = oracle.pack_canonical(q)
    tile = bl.import_canonical(dev(canon))
    assert_exact(host(tile), oracle.pack(q), "canonical -> tile")
    assert_exact(host(bl.export_canonical(tile)), canon, "tile -> canonical")
    assert_exact(host(bl.unpack_weights(tile)), q, "tile -> int8")
    p, s = gpu_pack(W)
    if host(s)[0] == g:
        assert_exact(host(bl.export_canonical(p)), canon, "packer output -> canonical")
        assert_exact(host(bl.unpack_weights(p)), q, "packer output -> int8")


def test_canonical_layout_hand_bytes(golden):
    """The hand-worked 2 x 4 matrix's plain bytes 0x16, 0x89, padded to K = 64
    with zero weights (code 1, bytes 0x55), through import and unpack."""
    gd = golden("hand_bitlinear_2x4.json")
    canon = np.full((2, 16), 0x55, np.uint8)
    canon[:, 0] = np.array(gd["packed_canonical"], np.uint8)[:, 0]
    q = np.zeros((2, 64), np.int8)
    q[:, :4] = np.array(gd["q"], np.int8)
    got = host(bl.unpack_weights(bl.import_canonical(dev(canon))))
    assert_exact(got, q, "hand bytes -> int8")


def test_inplace_quant_forward_rejected():
    """Y over X in the fused quantise + BitLinear (K == N, as in an in-place
    hidden update) is refused before anything runs; the input is untouched."""
    rng = np.random.default_rng(31)
    W = synth.weights(rng, 256, 256)
    p, s = gpu_pack(W)
    X = dev(synth.activations(rng, 2, 256))
    before = host(X).copy()
    with pytest.raises(bl.BitLinearError) as e:
        bl.quant_forward(X, p, s, y_out=X)
    assert e.value.status == bl.BL_ERR_UNSUPPORTED
    assert_exact(host(X), before, "X after a rejected call")


# ------------------------------------------------------------------ activation quantiser

@pytest.mark.parametrize("M,K,rms,gain", [(4, 256, False, False), (1, 2560, False, False),
                                          (37, 6912, True, True), (3, 16384, True, False),
                                          (5, 64, False, False), (9, 2560, True, False),
                                          (2, 8192, True, True), (2, 8256, False, False),
                                          (2, 16448, True, False), (2, 32768, False, False),
                                          (3, 32768, True, True)])
def test_quant(M, K, rms, gain):
    log(f"[quant] M={M} K={K} rms={rms} gain={gain}")
    rng = np.random.default_rng(M * 1000 + K)
    X = synth.activations(rng, M, K, outliers=True)
    g = synth.gains(rng, K) if gain else None
    xq, xs, rs = bl.quant_act(dev(X), rmsnorm=rms, norm_gain=None if g is None else dev(g))
    if rms:
        # RMSNorm first: its binary64 sum runs in another order on the GPU, so
        # a value at a rounding midpoint may flip (R3, teacher-forced)
        check_requant(oracle.rmsnorm(X, g), host(xq), host(xs), host(rs), f"quant M={M} K={K}")
    else:
        # the same binary32 products on both sides: bit-exact (R1)
        ref_q, ref_s, ref_r = oracle.quant_act(X)
        assert_exact(host(xq), ref_q, "xq")
        assert_exact(host(xs), ref_s, "scale")
        assert_exact(host(rs), ref_r, "rowsum")


def test_quant_edge_rows():
    X = np.zeros((4, 128), np.float32)
    X[1, 3] = 1e-7                                  # below the 1e-5 floor
    X[2, :] = -2.5                                  # constant row
    X[3, :8] = [2.5, -127, 0.5, -3.5, 1.5, 126.5, 0, -0.5]  # ties at scale 1
    log("[quant] edge rows")
    xq, xs, rs = bl.quant_act(dev(X))
    ref_q, ref_s, ref_r = oracle.quant_act(X)
    assert_exact(host(xq), ref_q, "edge xq")
    assert_exact(host(xs), ref_s, "edge scale")
    assert_exact(host(rs), ref_r, "edge rowsum")


# ------------------------------------------------------------------ forward

def run_forward(X, W, **kw):
    p, s, q, g = check_pack(W, "fwd")
    xq, xs, rs = bl.quant_act(dev(X))
    out = bl.forward(xq, xs, p, s, x_rowsum=rs, want_acc=True, **kw)
    ref = oracle.bitlinear(X, q, g)
    assert_exact(host(xq), ref["xq"], "xq")
    assert_exact(host(out["acc"]), ref["acc"], "acc")
    return out, ref, (xq, xs, rs, p, s, q, g)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 8, 9, 16, 17, 40, 64, 65, 130])
@pytest.mark.parametrize("K,N", [(256, 512), (192, 100), (2560, 200), (6912, 72), (64, 96), (128, 130), (320, 160)])
def test_forward_small(M, K, N):
    """One BitLinear from int8 rows against the oracle: up to 8 tokens the
    batched kernel copies half its token tile, 9..16 the whole tile, then
    two and four token tiles, and the GEMM beyond 64 tokens."""
    log(f"[forward] M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 31 + K + N)
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    out, ref, _ = run_forward(X, W)
    assert_y_close(host(out["y"]), ref["y"])


@pytest.mark.parametrize("M", [24, 48, 64])
@pytest.mark.parametrize("K,N,epi", [(1536, 4100, "residual"), (3584, 4098, "mul"), (5120, 200, "none"),
                                     (6016, 96, "residual"), (8192, 64, "none")])
def test_forward_batched_shapes(M, K, N, epi):
    """The batched-decode kernel (int8 rows, 17 <= M <= 64) at every chunk-quad
    count per wave from 2 to 8 (K = 1536 .. 8192), two column tiles per
    workgroup with N not a multiple of 32 (and, at N = 4098, rows that are not
    16-byte aligned: the element-wise epilogue), and the residual or gating
    epilogue operand; accumulators and outputs element by element."""
    log(f"[batched] M={M} K={K} N={N} epi={epi}")
    rng = np.random.default_rng(M * 7 + K + N)
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    aux = rng.standard_normal((M, N)).astype(np.float32)
    p, s, q, g = check_pack(W, "batched")
    xq, xs, rs = bl.quant_act(dev(X))
    kw = {}
    if epi == "residual":
        kw = {"residual": dev(aux)}
    elif epi == "mul":
        kw = {"mul_by": dev(aux)}
    out = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, want_acc=True, **kw)
    rq = oracle.quant_act(X)
    assert_exact(host(xq), rq[0], "xq")
    acc = oracle.int_matmul(rq[0], q)
    assert_exact(host(out["acc"]), acc, "acc")
    y = oracle.relu2(oracle.dequant(acc, rq[1], g))
    if epi == "residual":
        y = oracle.add(aux, y)
    elif epi == "mul":
        y = oracle.mul(y, aux)
    assert_y_close(host(out["y"]), y, "y")


def test_forward_rowsum_computed_inside():
    rng = np.random.default_rng(11)
    X = synth.activations(rng, 6, 512)
    W = synth.weights(rng, 300, 512)
    p, s, q, g = check_pack(W, "rowsum")
    xq, xs, rs = bl.quant_act(dev(X))
    a = bl.forward(xq, xs, p, s, x_rowsum=rs, want_acc=True)
    b = bl.forward(xq, xs, p, s, x_rowsum=None, want_acc=True)
    assert_exact(host(a["acc"]), host(b["acc"]), "acc with/without rowsum")
    assert_exact(host(a["y"]), host(b["y"]), "y with/without rowsum")


@pytest.mark.parametrize("M", [1, 4, 48])
def test_forward_relu2_residual(M):
    log(f"[forward epi] M={M}")
    rng = np.random.default_rng(500 + M)
    K, N = 1024, 320
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    R = synth.activations(rng, M, N)
    out, ref, (xq, xs, rs, p, s, q, g) = run_forward(X, W, relu2=True, residual=dev(R))
    assert_y_close(host(out["y"]), oracle.add(R, oracle.relu2(ref["y"])))
    # in place: Y aliases the residual
    h = dev(R)
    bl.forward(xq, xs, p, s, x_rowsum=rs, residual=h, y_out=h)
    assert_y_close(host(h), oracle.add(R, ref["y"]), "in-place residual")


@pytest.mark.parametrize("M,with_gain", [(1, False), (3, True), (40, True)])
def test_forward_subln_requant(M, with_gain):
    log(f"[forward subln] M={M}")
    rng = np.random.default_rng(700 + M)
    K, N = 640, 1536
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    gain = synth.gains(rng, N) if with_gain else None
    out, ref, _ = run_forward(X, W, relu2=True, subln=True,
                              norm_gain=None if gain is None else dev(gain))
    y = host(out["y"])
    assert_y_close(y, oracle.relu2(ref["y"]))
    # teacher-forced: the oracle normalises the GPU's own ReLU^2 output
    check_requant(oracle.rmsnorm(y, gain), host(out["q"]), host(out["q_scale"]), host(out["q_rowsum"]),
                  "subln")
    # without Y the requantised result is the same
    xq, xs, rs = bl.quant_act(dev(X))
    p, s = gpu_pack(W)
    o2 = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, subln=True, want_y=False,
                    norm_gain=None if gain is None else dev(gain))
    assert "y" not in o2
    assert_exact(host(o2["q"]), host(out["q"]), "subln without Y")


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 12])
@pytest.mark.parametrize("K,N,rms,gain,relu2,res", [(2560, 6912, False, False, True, False),
                                                     (6912, 2560, True, True, False, True),
                                                     (256, 512, True, False, False, False),
                                                     (640, 37, False, False, True, True),
                                                     (32768, 96, True, True, True, True)])
def test_quant_forward(M, K, N, rms, gain, relu2, res):
    """Fused quantise + BitLinear (one launch for M <= 4) against the oracle;
    at the widest supported row (K = 32768) the quantiser runs 1024 threads
    per row and the contraction goes to the GEMM whatever M."""
    log(f"[quant_forward] M={M} K={K} N={N} rms={rms} gain={gain} relu2={relu2} res={res}")
    rng = np.random.default_rng(M * 7 + K + N)
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    g = synth.gains(rng, K) if gain else None
    R = synth.activations(rng, M, N)
    p, s, q, gw = check_pack(W, "quant_forward")
    y = bl.quant_forward(dev(X), p, s, rmsnorm=rms, norm_gain=None if g is None else dev(g), relu2=relu2,
                         residual=dev(R) if res else None)
    z = oracle.rmsnorm(X, g) if rms else X
    xq, gx, _ = oracle.quant_act(z)
    want = oracle.dequant(oracle.int_matmul(xq, q), gx, gw)
    if relu2:
        want = oracle.relu2(want)
    if res:
        want = oracle.add(R, want)
    assert_y_close(host(y), want, "quant_forward y")
    # same values as the two-step path on the GPU
    xq2, xs2, rs2 = bl.quant_act(dev(X), rmsnorm=rms, norm_gain=None if g is None else dev(g))
    two = bl.forward(xq2, xs2, p, s, x_rowsum=rs2, relu2=relu2, residual=dev(R) if res else None)
    assert_exact(host(y), host(two["y"]), "quant_forward vs quant_act + forward")
    if res:  # in place
        h = dev(R)
        bl.quant_forward(dev(X), p, s, rmsnorm=rms, norm_gain=None if g is None else dev(g), relu2=relu2,
                         residual=h, y_out=h)
        assert_exact(host(h), host(y), "quant_forward in place")


@pytest.mark.parametrize("M", [1, 4, 8, 17, 33, 64, 80])
def test_forward_grouped(M):
    """Grouped BitLinears on one set of int8 rows: q, k, v shapes (2560 ->
    2560, 640, 640, each with its own absmean scale) plus a ragged matrix,
    with ReLU^2, residual, gating product and subln requantisation spread over
    the matrices: every output bit-identical to one bitlinear_forward per
    matrix (one launch for M <= 64, one per matrix beyond), and against the
    oracle."""
    log(f"[grouped] M={M}")
    rng = np.random.default_rng(3300 + M)
    K = 2560
    X = synth.activations(rng, M, K, outliers=True)
    shapes = [(2560, {"relu2": True, "subln": True}), (640, {"residual": True}), (640, {"mul": True}),
              (200, {})]
    packs, mats, refs = [], [], []
    xq, xs, rs = bl.quant_act(dev(X))
    rq = oracle.quant_act(X)
    assert_exact(host(xq), rq[0], "xq")
    for i, (N, kw) in enumerate(shapes):
        W = synth.weights(rng, N, K)
        p, s, q, g = check_pack(W, f"grouped {i}")
        A = synth.activations(rng, M, N)
        d = {"packed": p, "w_scale": s, "want_acc": True, "relu2": kw.get("relu2", False),
             "subln": kw.get("subln", False)}
        if kw.get("residual"):
            d["residual"] = dev(A)
        if kw.get("mul"):
            d["mul_by"] = dev(A)
        mats.append(d)
        packs.append((p, s, q, g, A, kw))
    out = bl.forward_grouped(xq, xs, rs, mats)
    for i, (p, s, q, g, A, kw) in enumerate(packs):
        one = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=kw.get("relu2", False), subln=kw.get("subln", False),
                         residual=dev(A) if kw.get("residual") else None,
                         mul_by=dev(A) if kw.get("mul") else None, want_acc=True)
        for key in one:
            assert_exact(host(out[i][key]), host(one[key]), f"matrix {i} {key}: grouped vs single")
        acc = oracle.int_matmul(rq[0], q)
        assert_exact(host(out[i]["acc"]), acc, f"matrix {i} acc")
        want = oracle.dequant(acc, rq[1], g)
        if kw.get("relu2"):
            want = oracle.relu2(want)
        if kw.get("residual"):
            want = oracle.add(A, want)
        if kw.get("mul"):
            want = oracle.mul(want, A)
        assert_y_close(host(out[i]["y"]), want, f"matrix {i} y")
        if kw.get("subln"):
            check_requant(oracle.rmsnorm(host(out[i]["y"])), host(out[i]["q"]), host(out[i]["q_scale"]),
                          host(out[i]["q_rowsum"]), f"matrix {i} subln")


def _stationary_cases():
    # (M, K, row counts of the matrices): at least 512 tiles of 16 rows, so the
    # launch copies all activations into LDS once per workgroup; ragged N, K
    # with a partial last chunk quad and K % 128 == 64 (unswizzled tail)
    # (up to 32 tokens); beyond 32 tokens the same calls run k_batch, with
    # four column tiles per workgroup once that still fills every CU (ragged
    # matrices whose last workgroup has empty column tiles, K = 6912)
    return [(1, 2560, (2560, 6912, 6912)), (5, 576, (3000, 3001, 2999)), (16, 64, (8200,)),
            (17, 1088, (4100, 4099)), (31, 1344, (600, 7700, 5)), (32, 2560, (2560, 6912, 6912)),
            (33, 2560, (2560, 6912, 6912)), (48, 192, (9000,)), (64, 2560, (2560, 6912, 6912)),
            (40, 1088, (4100, 4099, 8200)), (36, 6912, (16400,))]


@pytest.mark.parametrize("M,K,Ns", _stationary_cases())
def test_forward_stationary(M, K, Ns):
    """The activation-stationary launch (many 16-row tiles, K <= 2560): int32
    accumulators bit-exact and outputs within 1e-5 of the oracle for every
    matrix, with ReLU^2, residual and gating product epilogues; the same
    values as the matrices run one by one through the grouped call's
    per-matrix path is implied by the oracle match."""
    log(f"[stationary] M={M} K={K} N={Ns}")
    rng = np.random.default_rng(3400 + M + K)
    X = synth.activations(rng, M, K, outliers=True)
    xq, xs, rs = bl.quant_act(dev(X))
    rq = oracle.quant_act(X)
    epis = [{"relu2": True}, {"residual": True}, {"mul": True}, {}]
    mats, refs = [], []
    for i, N in enumerate(Ns):
        W = synth.weights(rng, N, K)
        p, s, q, g = check_pack(W, f"stationary {i}")
        A = synth.activations(rng, M, N)
        kw = epis[i % len(epis)]
        d = {"packed": p, "w_scale": s, "want_acc": True, "relu2": kw.get("relu2", False)}
        if kw.get("residual"):
            d["residual"] = dev(A)
        if kw.get("mul"):
            d["mul_by"] = dev(A)
        mats.append(d)
        refs.append((q, g, A, kw))
    out = bl.forward_grouped(xq, xs, rs, mats) if len(Ns) > 1 else [bl.forward(
        xq, xs, mats[0]["packed"], mats[0]["w_scale"], x_rowsum=rs, want_acc=True, relu2=mats[0]["relu2"])]
    for i, (q, g, A, kw) in enumerate(refs):
        with oracle.parallel():
            acc = oracle.int_matmul(rq[0], q)
        assert_exact(host(out[i]["acc"]), acc, f"matrix {i} acc")
        want = oracle.dequant(acc, rq[1], g)
        if kw.get("relu2"):
            want = oracle.relu2(want)
        if kw.get("residual"):
            want = oracle.add(A, want)
        if kw.get("mul"):
            want = oracle.mul(want, A)
        assert_y_close(host(out[i]["y"]), want, f"matrix {i} y")


def _quant_grouped_cases():
    # (M, K, row counts of the matrices, RMSNorm, gain): the launch that
    # quantises its rows itself (up to 8 tokens, at least 512 tiles of 16
    # rows, K <= 2560), with and without RMSNorm and gain, K with a partial
    # last float4 group of the 256-thread quantiser and a partial chunk quad;
    # then the two-step path (9 tokens, too few tiles, K above 2560)
    return [(1, 2560, (2560, 6912, 6912), False, False), (8, 2560, (2560, 6912, 6912), False, False),
            (3, 2560, (2560, 6912, 6912), True, True), (5, 576, (3000, 3001, 2999), True, False),
            (7, 1088, (4100, 4099), True, True), (2, 64, (8200,), False, False),
            (9, 2560, (2560, 6912, 6912), True, True), (4, 2560, (640, 640), False, False),
            (8, 2624, (8200,), True, True)]


@pytest.mark.parametrize("M,K,Ns,rms,gain", _quant_grouped_cases())
def test_quant_forward_grouped(M, K, Ns, rms, gain):
    """bitlinear_quant_forward_grouped: every output (y, acc, subln requant)
    bit-identical to bitlinear_quant_act followed by
    bitlinear_forward_grouped, with ReLU^2, residual, gating product and
    subln epilogues; the quantised rows themselves against the oracle (R1
    without RMSNorm, R3 with it)."""
    log(f"[quant grouped] M={M} K={K} N={Ns} rms={rms} gain={gain}")
    rng = np.random.default_rng(3500 + M + K + 2 * rms + gain)
    X = synth.activations(rng, M, K, outliers=True)
    G = synth.gains(rng, K) if gain else None
    gdev = None if G is None else dev(G)
    epis = [{"relu2": True, "subln": True}, {"residual": True}, {"mul": True}, {}]
    mats = []
    for i, N in enumerate(Ns):
        p, s = gpu_pack(synth.weights(rng, N, K))
        kw = epis[i % len(epis)]
        d = {"packed": p, "w_scale": s, "want_acc": True, "relu2": kw.get("relu2", False),
             "subln": kw.get("subln", False) and N % 64 == 0}
        if d["subln"]:
            d["norm_gain"] = dev(synth.gains(rng, N))
        if kw.get("residual"):
            d["residual"] = dev(synth.activations(rng, M, N))
        if kw.get("mul"):
            d["mul_by"] = dev(synth.activations(rng, M, N))
        mats.append(d)
    xq, xs, rs = bl.quant_act(dev(X), rmsnorm=rms, norm_gain=gdev)
    want = bl.forward_grouped(xq, xs, rs, mats)
    got = bl.quant_forward_grouped(dev(X), mats, rmsnorm=rms, norm_gain=gdev)
    for i in range(len(Ns)):
        assert set(got[i]) == set(want[i])
        for key in want[i]:
            assert_exact(host(got[i][key]), host(want[i][key]), f"matrix {i} {key}: fused vs two calls")
    if rms:
        check_requant(oracle.rmsnorm(X, G), host(xq), host(xs), host(rs), f"quant grouped M={M} K={K}")
    else:
        ref_q, ref_s, ref_r = oracle.quant_act(X)
        assert_exact(host(xq), ref_q, "xq")
        assert_exact(host(xs), ref_s, "scale")
        assert_exact(host(rs), ref_r, "rowsum")


def test_gemv_row_equals_gemm_row():
    """Token independence across kernels: M=1 (batched kernel, one token tile) equals
    row 0 of M=80 (tiled GEMM)."""
    rng = np.random.default_rng(21)
    X = synth.activations(rng, 80, 2560, outliers=True)
    W = synth.weights(rng, 640, 2560)
    p, s = gpu_pack(W)
    xq, xs, rs = bl.quant_act(dev(X))
    full = bl.forward(xq, xs, p, s, x_rowsum=rs, want_acc=True)
    one = bl.forward(xq[:1].contiguous(), xs[:1].contiguous(), p, s, x_rowsum=rs[:1].contiguous(),
                     want_acc=True)
    assert_exact(host(one["acc"])[0], host(full["acc"])[0], "gemv vs gemm acc")
    assert_exact(host(one["y"])[0], host(full["y"])[0], "gemv vs gemm y")


def test_determinism():
    rng = np.random.default_rng(22)
    X = synth.activations(rng, 64, 2560)
    W = synth.weights(rng, 1024, 2560)
    p, s = gpu_pack(W)
    p2, s2 = gpu_pack(W)
    assert_exact(host(p2), host(p), "pack twice")
    xq, xs, rs = bl.quant_act(dev(X), rmsnorm=True)
    a = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, subln=True)
    b = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, subln=True)
    for k in ("y", "q", "q_scale", "q_rowsum"):
        assert_exact(host(a[k]), host(b[k]), f"twice: {k}")


# ------------------------------------------------------------------ FFN block

def ffn_layers_np(rng, n, H, F, gains=False):
    out = []
    for _ in range(n):
        Wu = synth.weights(rng, F, H)
        Wd = synth.weights(rng, H, F)
        pre = synth.gains(rng, H) if gains else None
        sub = synth.gains(rng, F) if gains else None
        out.append((Wu, Wd, pre, sub))
    return out


def to_gpu_layers(layers_np):
    gl, ol = [], []
    for Wu, Wd, pre, sub in layers_np:
        pu, su, qu, gu = check_pack(Wu, "ffn up")
        pd, sd, qd, gd = check_pack(Wd, "ffn down")
        gl.append({"up": pu, "up_scale": su, "down": pd, "down_scale": sd,
                   "pre_norm_gain": None if pre is None else dev(pre),
                   "sub_norm_gain": None if sub is None else dev(sub)})
        ol.append({"q_up": qu, "gamma_up": gu, "q_down": qd, "gamma_down": gd,
                   "pre_gain": pre if pre is not None else np.ones(Wu.shape[1], np.float32),
                   "sub_gain": sub})
    return gl, ol


def layer_teacher_forced(h_in, gpu_layer, ora_layer, M, pre=True, residual=True):
    """One layer on the GPU, checked stage by stage against the oracle fed with
    the GPU's own stage inputs.  Returns (gpu output, explained flips)."""
    H = h_in.shape[1]
    flips = 0
    x = dev(h_in)
    pre_g = gpu_layer["pre_norm_gain"]
    xq, xs, rs = bl.quant_act(x, rmsnorm=pre, norm_gain=pre_g)
    z = oracle.rmsnorm(h_in, ora_layer["pre_gain"]) if pre else h_in
    flips += check_requant(z, host(xq), host(xs), host(rs), "ffn input quant")
    up = bl.forward(xq, xs, gpu_layer["up"], gpu_layer["up_scale"], x_rowsum=rs, relu2=True, subln=True,
                    norm_gain=gpu_layer["sub_norm_gain"], want_acc=True)
    acc1 = oracle.int_matmul(host(xq), ora_layer["q_up"])
    assert_exact(host(up["acc"]), acc1, "ffn up acc")
    y1 = host(up["y"])
    assert_y_close(y1, oracle.relu2(oracle.dequant(acc1, host(xs), ora_layer["gamma_up"])), "ffn up y")
    flips += check_requant(oracle.rmsnorm(y1, ora_layer["sub_gain"]), host(up["q"]), host(up["q_scale"]),
                           host(up["q_rowsum"]), "ffn subln")
    h = dev(h_in)
    dn = bl.forward(up["q"], up["q_scale"], gpu_layer["down"], gpu_layer["down_scale"], x_rowsum=up["q_rowsum"],
                    residual=h if residual else None, y_out=h, want_acc=True)
    acc2 = oracle.int_matmul(host(up["q"]), ora_layer["q_down"])
    assert_exact(host(dn["acc"]), acc2, "ffn down acc")
    y2 = oracle.dequant(acc2, host(up["q_scale"]), ora_layer["gamma_down"])
    want = oracle.add(h_in, y2) if residual else y2
    assert_y_close(host(h), want, "ffn down y")
    return host(h), flips


@pytest.mark.parametrize("M", [1, 3, 20])
def test_ffn_block_small(M):
    log(f"[ffn] M={M}")
    rng = np.random.default_rng(900 + M)
    H, F, L = 256, 640, 3
    gl, ol = to_gpu_layers(ffn_layers_np(rng, L, H, F, gains=True))
    h0 = synth.activations(rng, M, H)
    # stage by stage, teacher forced
    h = h0
    for l in range(L):
        h, _ = layer_teacher_forced(h, gl[l], ol[l], M)
    # the stack call (fused decode kernels for M <= 4) gives exactly the
    # staged calls' results: same quantiser reductions, exact integer sums
    hs = dev(h0)
    stack = bl.FFNStack(gl, H, F, M, DEV)
    stack(hs)
    assert_exact(host(hs), h, "ffn stack vs staged calls")
    # twice in a row on the same workspace: same result
    hs2 = dev(h0)
    stack(hs2)
    assert_exact(host(hs2), h, "ffn stack, second call")
    # free running against the oracle stack (information, loose bound)
    ref = oracle.ffn_stack(h0, ol)
    assert np.abs(host(hs) - ref).max() <= 1e-3 * np.abs(ref).max()


@pytest.mark.parametrize("M,H,F", [(1, 256, 32768), (5, 32768, 256), (70, 128, 32768)])
def test_ffn_max_width(M, H, F):
    """FFN layers at the widest supported rows (32768): the 1024-thread
    quantiser on the intermediate row (subln) or on the hidden row (pre-norm),
    the down projection's K = 32768 or its 32768 outputs, checked stage by
    stage against the oracle; the stack call equals the staged calls."""
    log(f"[ffn max width] M={M} H={H} F={F}")
    rng = np.random.default_rng(980 + M)
    gl, ol = to_gpu_layers(ffn_layers_np(rng, 2, H, F, gains=True))
    h0 = synth.activations(rng, M, H, outliers=True)
    h = h0
    for l in range(2):
        h, _ = layer_teacher_forced(h, gl[l], ol[l], M)
    hs = dev(h0)
    bl.FFNStack(gl, H, F, M, DEV)(hs)
    assert_exact(host(hs), h, "ffn max width: stack vs staged calls")


def test_ffn_no_prenorm_no_residual():
    rng = np.random.default_rng(950)
    H, F = 128, 256
    gl, ol = to_gpu_layers(ffn_layers_np(rng, 1, H, F))
    h0 = synth.activations(rng, 5, H, outliers=True)
    h, _ = layer_teacher_forced(h0, gl[0], ol[0], 5, pre=False, residual=False)
    hs = dev(h0)
    bl.ffn_forward(gl, hs, pre_norm=False, residual=False)
    assert_exact(host(hs), h, "ffn flags=0")


# ------------------------------------------------------------------ gating product, gated FFN

@pytest.mark.parametrize("M", [1, 3, 12, 70, 130])
@pytest.mark.parametrize("K,N", [(256, 512), (320, 130)])
def test_forward_mul_epilogue(M, K, N):
    """y = ReLU^2(dequant(acc)) * aux, written in place over aux, through the
    batched (M <= 64) and GEMM paths; the fused quantise + forward (M <= 4
    one launch) gives the same values."""
    log(f"[mul epilogue] M={M} K={K} N={N}")
    rng = np.random.default_rng(M * 13 + K + N)
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    aux = rng.standard_normal((M, N)).astype(np.float32)
    p, s, q, g = check_pack(W, "mul")
    xq, xs, rs = bl.quant_act(dev(X))
    a = dev(aux)
    out = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, mul_by=a, y_out=a, want_acc=True)
    rq = oracle.quant_act(X)
    acc = oracle.int_matmul(rq[0], q)
    assert_exact(host(out["acc"]), acc, "acc")
    assert_y_close(host(a), oracle.mul(oracle.relu2(oracle.dequant(acc, rq[1], g)), aux), "relu2 * aux")
    if M <= 12:
        a2 = dev(aux)
        bl.quant_forward(dev(X), p, s, relu2=True, mul_by=a2, y_out=a2)
        assert_exact(host(a2), host(a), "quant_forward vs forward")


def gated_layers_np(rng, n, H, F, gains=False):
    out = []
    for _ in range(n):
        Wg = synth.weights(rng, F, H)
        Wu = synth.weights(rng, F, H)
        Wd = synth.weights(rng, H, F)
        pre = synth.gains(rng, H) if gains else None
        sub = synth.gains(rng, F) if gains else None
        out.append((Wg, Wu, Wd, pre, sub))
    return out


def to_gpu_gated(layers_np):
    gl, ol = [], []
    for Wg, Wu, Wd, pre, sub in layers_np:
        pg, sg, qg, gg = check_pack(Wg, "ffn gate")
        pu, su, qu, gu = check_pack(Wu, "ffn up")
        pd, sd, qd, gd = check_pack(Wd, "ffn down")
        gl.append({"gate": pg, "gate_scale": sg, "up": pu, "up_scale": su, "down": pd, "down_scale": sd,
                   "pre_norm_gain": None if pre is None else dev(pre),
                   "sub_norm_gain": None if sub is None else dev(sub)})
        ol.append({"q_gate": qg, "gamma_gate": gg, "q_up": qu, "gamma_up": gu, "q_down": qd, "gamma_down": gd,
                   "pre_gain": pre if pre is not None else np.ones(Wu.shape[1], np.float32), "sub_gain": sub})
    return gl, ol


def gated_layer_teacher_forced(h_in, G, O, pre=True, residual=True):
    """One gated layer through the C ABI stage by stage (up, then gate with
    ReLU^2 * up and the subln requantisation, then down), each stage against
    the oracle fed with the GPU's inputs to it.  Returns (output, flips)."""
    flips = 0
    xq, xs, rs = bl.quant_act(dev(h_in), rmsnorm=pre, norm_gain=G["pre_norm_gain"])
    z = oracle.rmsnorm(h_in, O["pre_gain"]) if pre else h_in
    flips += check_requant(z, host(xq), host(xs), host(rs), "gated input quant")
    up = bl.forward(xq, xs, G["up"], G["up_scale"], x_rowsum=rs, want_acc=True)
    acc_u = oracle.int_matmul(host(xq), O["q_up"])
    assert_exact(host(up["acc"]), acc_u, "gated up acc")
    yu = host(up["y"])
    assert_y_close(yu, oracle.dequant(acc_u, host(xs), O["gamma_up"]), "gated up y")
    gt = bl.forward(xq, xs, G["gate"], G["gate_scale"], x_rowsum=rs, relu2=True, mul_by=up["y"], subln=True,
                    norm_gain=G["sub_norm_gain"], want_acc=True)
    acc_g = oracle.int_matmul(host(xq), O["q_gate"])
    assert_exact(host(gt["acc"]), acc_g, "gate acc")
    hh = host(gt["y"])
    assert_y_close(hh, oracle.mul(oracle.relu2(oracle.dequant(acc_g, host(xs), O["gamma_gate"])), yu), "gated h")
    flips += check_requant(oracle.rmsnorm(hh, O["sub_gain"]), host(gt["q"]), host(gt["q_scale"]),
                           host(gt["q_rowsum"]), "gated subln")
    h = dev(h_in)
    dn = bl.forward(gt["q"], gt["q_scale"], G["down"], G["down_scale"], x_rowsum=gt["q_rowsum"],
                    residual=h if residual else None, y_out=h, want_acc=True)
    acc2 = oracle.int_matmul(host(gt["q"]), O["q_down"])
    assert_exact(host(dn["acc"]), acc2, "gated down acc")
    y2 = oracle.dequant(acc2, host(gt["q_scale"]), O["gamma_down"])
    assert_y_close(host(h), oracle.add(h_in, y2) if residual else y2, "gated down y")
    return host(h), flips


@pytest.mark.parametrize("M", [1, 3, 8, 20, 33, 64])
def test_ffn_gated_block(M):
    """Gated FFN layers (ReLU^2(gate) * up): teacher-forced stage by stage,
    then the stack call (gate and up in one launch: the decode kernel for
    M <= 4, the batched kernel up to 64, then the staged kernels) exactly
    equal to the staged calls, twice in a row."""
    log(f"[ffn gated] M={M}")
    rng = np.random.default_rng(1900 + M)
    H, F, L = 256, 640, 2
    gl, ol = to_gpu_gated(gated_layers_np(rng, L, H, F, gains=True))
    h0 = synth.activations(rng, M, H)
    h = h0
    for l in range(L):
        h, _ = gated_layer_teacher_forced(h, gl[l], ol[l])
    stack = bl.FFNStack(gl, H, F, M, DEV)
    for rep in range(2):
        hs = dev(h0)
        stack(hs)
        assert_exact(host(hs), h, f"gated stack vs staged calls (call {rep})")
    ref = h0
    for O in ol:
        ref = oracle.ffn_layer_gated(ref, O["q_gate"], O["gamma_gate"], O["q_up"], O["gamma_up"], O["q_down"],
                                     O["gamma_down"], pre_gain=O["pre_gain"], sub_gain=O["sub_gain"])
    assert np.abs(host(hs) - ref).max() <= 1e-3 * np.abs(ref).max()


@pytest.mark.parametrize("M", [16, 64])
def test_ffn_gated_model_width(M):
    """A gated layer at hidden 2560 / intermediate 6912 with gains, pre-norm
    and residual, M = 16 and 64 (one batched launch streams gate and up):
    exactly the staged calls, and the staged calls against the oracle."""
    log(f"[ffn gated, model width] M={M}")
    rng = np.random.default_rng(2700 + M)
    gl, ol = to_gpu_gated(gated_layers_np(rng, 1, synth.HIDDEN, synth.FFN, gains=True))
    h0 = synth.activations(rng, M, synth.HIDDEN)
    h, _ = gated_layer_teacher_forced(h0, gl[0], ol[0])
    hs = dev(h0)
    bl.FFNStack(gl, synth.HIDDEN, synth.FFN, M, DEV)(hs)
    assert_exact(host(hs), h, "gated stack vs staged calls")


# ------------------------------------------------------------------ very tall matrices at decode

@pytest.mark.parametrize("M,K,N,epi", [(1, 2560, 40008, "relu2"), (3, 256, 33000, "residual"),
                                        (4, 512, 32768, "none"), (2, 1024, 36880, "mul"),
                                        (1, 256, 200_008, "relu2"), (2, 6912, 32776, "residual")])
def test_decode_tall(M, K, N, epi):
    """At 2048 or more 16-row tiles the fused quantise + BitLinear launch
    is persistent: each workgroup quantises the rows once and walks groups
    of tiles (many per workgroup at N = 200,008), the last group ragged or
    partly empty: Y against the oracle, and bit for bit against the two-step
    path (quantiser + batched kernel)."""
    log(f"[decode tall] M={M} K={K} N={N} epi={epi}")
    rng = np.random.default_rng(7000 + M + N)
    X = synth.activations(rng, M, K, outliers=True)
    W = synth.weights(rng, N, K)
    A = synth.activations(rng, M, N)
    p, s, q, gw = check_pack(W, "decode tall")
    kw = dict(relu2=epi == "relu2", residual=dev(A) if epi == "residual" else None,
              mul_by=dev(A) if epi == "mul" else None)
    y = bl.quant_forward(dev(X), p, s, **kw)
    xq, gx, _ = oracle.quant_act(X)
    want = oracle.dequant(oracle.int_matmul(xq, q), gx, gw)
    if epi == "relu2":
        want = oracle.relu2(want)
    elif epi == "residual":
        want = oracle.add(A.copy(), want)
    elif epi == "mul":
        want = oracle.mul(want, A)
    assert_y_close(host(y), want, "tall decode y")
    a, b, r = bl.quant_act(dev(X))
    two = bl.forward(a, b, p, s, x_rowsum=r, **kw)
    assert_exact(host(y), host(two["y"]), "tall decode vs quantiser + batched kernel")


# ------------------------------------------------------------------ seeded shape sweep

def _sweep_cases(n=40, seed=6100):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.choice([1, 2, 3, 4, 5, 8, 13, 16, 17, 31, 33, 48, 64, 65, 100, 129, 200, 300]))
        K = 64 * int(rng.integers(1, 65))          # 64 .. 4096
        N = int(rng.integers(1, 3001))
        epi = str(rng.choice(["none", "relu2", "residual", "mul", "relu2+residual"]))
        cases.append((i, M, K, N, epi))
    return cases


@pytest.mark.parametrize("i,M,K,N,epi", _sweep_cases())
def test_forward_shape_sweep(i, M, K, N, epi):
    """40 seeded shapes over the decode (M <= 4), batched (M <= 64) and GEMM
    paths, ragged N, K up to 4096, with the epilogue flags: int32 acc bit-exact
    and Y within 1e-5 of the oracle; quant_forward equal to quant_act +
    forward bit for bit."""
    log(f"[sweep {i}] M={M} K={K} N={N} epi={epi}")
    rng = np.random.default_rng(6200 + i)
    X = synth.activations(rng, M, K, outliers=bool(i % 2))
    W = synth.weights(rng, N, K)
    A = synth.activations(rng, M, N)
    p, s, q, gw = check_pack(W, f"sweep {i}")
    relu2 = "relu2" in epi
    res = dev(A) if "residual" in epi else None
    mul = dev(A) if epi == "mul" else None
    xq, xs, rs = bl.quant_act(dev(X))
    out = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=relu2, residual=res, mul_by=mul, want_acc=True)
    oq, og, _ = oracle.quant_act(X)
    assert_exact(host(xq), oq, "sweep xq")
    acc = oracle.int_matmul(oq, q)
    assert_exact(host(out["acc"]), acc, "sweep acc")
    want = oracle.dequant(acc, og, gw)
    if relu2:
        want = oracle.relu2(want)
    if "residual" in epi:
        want = oracle.add(A.copy(), want)
    elif epi == "mul":
        want = oracle.mul(want, A)
    assert_y_close(host(out["y"]), want, "sweep y")
    y2 = bl.quant_forward(dev(X), p, s, relu2=relu2, residual=res, mul_by=mul)
    assert_exact(host(y2), host(out["y"]), "sweep quant_forward vs quant_act + forward")


@pytest.mark.parametrize("M,K,N", [(512, 256, 512), (2304, 64, 6912)])
def test_gemm_whole_tile_epilogues(M, K, N):
    """The GEMM path's whole tiles store Y through LDS staging; the int32
    accumulators are not requested here, so that path runs (asking for them
    takes the element-wise one).  512 x 512 runs 256x160 tiles, the last one
    partial; 2304 x 6912 runs 256x256 tiles, all whole.  Every epilogue:
    plain, ReLU^2, residual add and gating product, alone and after ReLU^2;
    Y within 1e-5 of the oracle."""
    log(f"[gemm tiles] M={M} K={K} N={N}")
    rng = np.random.default_rng(7300 + M)
    X = synth.activations(rng, M, K)
    W = synth.weights(rng, N, K)
    A = synth.activations(rng, M, N)
    p, s, q, gw = check_pack(W, "gemm tiles")
    xq, xs, rs = bl.quant_act(dev(X))
    oq, og, _ = oracle.quant_act(X)
    assert_exact(host(xq), oq, "gemm tiles xq")
    with oracle.parallel():
        acc = oracle.int_matmul(oq, q)
    base = oracle.dequant(acc, og, gw)
    aux = dev(A)
    for epi in ("none", "relu2", "residual", "mul", "relu2+residual", "relu2+mul"):
        relu2 = epi.startswith("relu2")
        res = aux if "residual" in epi else None
        mul = aux if "mul" in epi else None
        out = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=relu2, residual=res, mul_by=mul)
        want = oracle.relu2(base.copy()) if relu2 else base.copy()
        if res is not None:
            want = oracle.add(A.copy(), want)
        elif mul is not None:
            want = oracle.mul(want, A)
        assert_y_close(host(out["y"]), want, f"gemm tiles {epi}")


def _ffn_sweep_cases(n=12, seed=6300):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 4, 6, 19, 40, 64, 80, 150]))
        H = 64 * int(rng.integers(1, 25))
        F = 64 * int(rng.integers(1, 25))
        out.append((i, M, H, F, bool(rng.integers(0, 2)), bool(rng.integers(0, 2)), bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,M,H,F,gated,pre,residual", _ffn_sweep_cases())
def test_ffn_shape_sweep(i, M, H, F, gated, pre, residual):
    """12 seeded FFN layer shapes, plain and gated, with and without pre-norm
    and residual, across the decode, batched and GEMM paths: the stack call
    exactly equals the staged calls, which are checked stage by stage
    against the oracle."""
    log(f"[ffn sweep {i}] M={M} H={H} F={F} gated={gated} pre={pre} residual={residual}")
    rng = np.random.default_rng(6400 + i)
    if gated:
        gl, ol = to_gpu_gated(gated_layers_np(rng, 1, H, F, gains=True))
    else:
        gl, ol = to_gpu_layers(ffn_layers_np(rng, 1, H, F, gains=True))
    h0 = synth.activations(rng, M, H)
    if gated:
        h, _ = gated_layer_teacher_forced(h0, gl[0], ol[0], pre=pre, residual=residual)
    else:
        h, _ = layer_teacher_forced(h0, gl[0], ol[0], M, pre=pre, residual=residual)
    hs = dev(h0)
    bl.ffn_forward(gl, hs, pre_norm=pre, residual=residual)
    assert_exact(host(hs), h, "ffn sweep: stack vs staged calls")


# ------------------------------------------------------------------ forward from latent weights

def latent_weights(rng, N, K, dtype):
    """(device tensor in the given dtype, the same numbers as fp32 numpy)."""
    if dtype == "bf16":
        bits, W = synth.weights_bf16(rng, N, K)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16), W
    W = synth.weights(rng, N, K)
    return dev(W), W


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("M,K,N,epi", [(1, 256, 130, "relu2"), (3, 2560, 6912, None), (8, 320, 512, "residual"),
                                        (70, 512, 200, "mul"), (300, 1024, 272, "relu2"), (2, 512, 96, "rms"),
                                        (40, 768, 160, "rms")])
def test_latent_forward(M, K, N, epi, dtype):
    """BitLinear from latent fp32 / bf16 weights (ternarised inside the call)
    through the fused decode (M <= 4), batched and GEMM paths: gamma_w and Y
    exactly those of pack + quant_forward on the same numbers, Y against the
    oracle, and without an epilogue within 1e-6 of the binary64 fake-quant
    product of the dequantised operands."""
    log(f"[latent forward] M={M} K={K} N={N} epi={epi} {dtype}")
    rng = np.random.default_rng(4100 + M + K + N + (dtype == "bf16"))
    Wt, W = latent_weights(rng, N, K, dtype)
    X = synth.activations(rng, M, K, outliers=True)
    A = synth.activations(rng, M, N)
    G = synth.gains(rng, K)
    kw = dict(relu2=epi == "relu2", residual=dev(A) if epi == "residual" else None,
              mul_by=dev(A) if epi == "mul" else None, rmsnorm=epi == "rms",
              norm_gain=dev(G) if epi == "rms" else None)
    gw_t = torch.empty(1, dtype=torch.float32, device=DEV)
    y = bl.latent_forward(dev(X), Wt, w_scale_out=gw_t, **kw)
    p, s, q, gw = check_pack(W, "latent forward")
    assert host(gw_t)[0] == host(s)[0], "gamma_w of the latent forward vs the packer"
    y2 = bl.quant_forward(dev(X), p, s, **kw)
    assert_exact(host(y), host(y2), "latent forward vs pack + quant_forward")
    z = oracle.rmsnorm(X, G) if epi == "rms" else X
    if epi == "rms":  # the GPU's own quantised rows decide near-ties (same precision, explained flips)
        xq_g, xs_g, rs_g = bl.quant_act(dev(X), rmsnorm=True, norm_gain=dev(G))
        check_requant(z, host(xq_g), host(xs_g), host(rs_g), "latent forward rmsnorm quant")
    xq, gx, _ = oracle.quant_act(z)
    acc = oracle.int_matmul(xq, q)
    want = oracle.dequant(acc, gx, gw)
    if epi == "relu2":
        want = oracle.relu2(want)
    elif epi == "residual":
        want = oracle.add(A.copy(), want)
    elif epi == "mul":
        want = oracle.mul(want, A)
    assert_y_close(host(y), want, "latent forward y")
    if epi is None:
        fake = (xq.astype(np.float64) * (gx.astype(np.float64)[:, None] / 127.0)) @ \
            (q.astype(np.float64) * float(gw)).T
        scale = np.abs(fake).max(axis=1, keepdims=True)
        assert np.all(np.abs(host(y) - fake) <= 1e-6 * np.maximum(np.abs(fake), 1e-6 * scale))


def test_latent_forward_bf16_equals_f32_of_same_values():
    """bf16 latent weights give bit-identical results to the fp32 tensor of
    the same numbers (the widening is exact), at the model's up shape."""
    rng = np.random.default_rng(4200)
    bits, W = synth.weights_bf16(rng, synth.FFN, synth.HIDDEN)
    Wb = torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    X = dev(synth.activations(rng, 2, synth.HIDDEN, outliers=True))
    ya = bl.latent_forward(X, Wb, relu2=True)
    yb = bl.latent_forward(X, dev(W), relu2=True)
    assert_exact(host(ya), host(yb), "bf16 vs fp32 latent weights")
    assert torch.equal(Wb.float().cpu(), torch.from_numpy(W))  # torch's widening agrees


# ------------------------------------------------------------------ the five workloads

def test_workload_single_bitlinear():
    """M=4, K=256, N=512, seed 0: whole pipeline, every element."""
    d = synth.single_bitlinear()
    log("[workload] single bitlinear")
    out, ref, _ = run_forward(d["X"], d["W"])
    assert_y_close(host(out["y"]), ref["y"])


def test_workload_decode_gemv():
    """M=1 decode at model width: up 2560->6912 and down 6912->2560, seed 1:
    the staged calls, the fused quantise + BitLinear launches, and the FFN
    step exactly as the benchmark times it (bitnet_ffn_forward, M=1, no
    pre-norm, no residual: up + ReLU^2 with the rows quantised in every
    workgroup, then down with the subln requantisation fused), every element."""
    d = synth.decode_gemv()
    packs = {}
    for name in ("up", "down"):
        log(f"[workload] decode {name}")
        out, ref, (xq, xs, rs, p, s, q, g) = run_forward(d[f"X_{name}"], d[f"W_{name}"])
        assert_y_close(host(out["y"]), ref["y"])
        packs[name] = (p, s, q, g)
        y = bl.quant_forward(dev(d[f"X_{name}"]), p, s)
        assert_exact(host(y), host(out["y"]), f"decode {name}: fused vs staged")
    (pu, su, qu, gu), (pd, sd, qd, gd) = packs["up"], packs["down"]
    X = d["X_up"]
    h = dev(X)
    bl.FFNStack([{"up": pu, "up_scale": su, "down": pd, "down_scale": sd}], synth.HIDDEN, synth.FFN, 1, DEV,
                pre_norm=False, residual=False)(h)
    # teacher-forced: the staged calls, each against the oracle
    xq, xs, rs = bl.quant_act(dev(X))
    assert_exact(host(xq), oracle.quant_act(X)[0], "step xq")
    up = bl.forward(xq, xs, pu, su, x_rowsum=rs, relu2=True, subln=True, want_acc=True)
    acc1 = oracle.int_matmul(host(xq), qu)
    assert_exact(host(up["acc"]), acc1, "step up acc")
    y1 = host(up["y"])
    assert_y_close(y1, oracle.relu2(oracle.dequant(acc1, host(xs), gu)), "step up y")
    flips = check_requant(oracle.rmsnorm(y1), host(up["q"]), host(up["q_scale"]), host(up["q_rowsum"]),
                          "step subln")
    dn = bl.forward(up["q"], up["q_scale"], pd, sd, x_rowsum=up["q_rowsum"], want_acc=True)
    acc2 = oracle.int_matmul(host(up["q"]), qd)
    assert_exact(host(dn["acc"]), acc2, "step down acc")
    assert_y_close(host(dn["y"]), oracle.dequant(acc2, host(up["q_scale"]), gd), "step down y")
    assert_exact(host(h), host(dn["y"]), "benchmarked FFN step vs staged calls")
    # free running (information): the oracle's own chain from X
    ref, _ = oracle.ffn_layer(X, qu, gu, qd, gd, pre_gain=None, residual=False, intermediates=True)
    log(f"[workload] decode step: near-tie flips {flips}, free-running max |diff| / max |y| = "
        f"{np.abs(host(h) - ref).max() / np.abs(ref).max():.3g}")


def test_workload_batched_decode():
    """M = 8, 32, 64: o, gate, up (+ReLU^2 + subln requant), down, seed 2."""
    d = synth.batched_decode()
    packs = {n: check_pack(d[f"W_{n}"], n) for n in ("o", "gate", "up", "down")}
    for M in (8, 32, 64):
        X = d[f"X{M}"]
        log(f"[workload] batched decode M={M}")
        xq, xs, rs = bl.quant_act(dev(X))
        ref_q = oracle.quant_act(X)
        assert_exact(host(xq), ref_q[0], "xq")
        for n in ("o", "gate"):
            p, s, q, g = packs[n]
            out = bl.forward(xq, xs, p, s, x_rowsum=rs, want_acc=True)
            acc = oracle.int_matmul(ref_q[0], q)
            assert_exact(host(out["acc"]), acc, f"{n} acc")
            assert_y_close(host(out["y"]), oracle.dequant(acc, ref_q[1], g), f"{n} y")
        p, s, q, g = packs["up"]
        up = bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, subln=True, want_acc=True)
        acc = oracle.int_matmul(ref_q[0], q)
        assert_exact(host(up["acc"]), acc, "up acc")
        y1 = host(up["y"])
        assert_y_close(y1, oracle.relu2(oracle.dequant(acc, ref_q[1], g)), "up y")
        flips = check_requant(oracle.rmsnorm(y1), host(up["q"]), host(up["q_scale"]), host(up["q_rowsum"]),
                              "subln")
        p, s, q, g = packs["down"]
        dn = bl.forward(up["q"], up["q_scale"], p, s, x_rowsum=up["q_rowsum"], want_acc=True)
        acc = oracle.int_matmul(host(up["q"]), q)
        assert_exact(host(dn["acc"]), acc, "down acc")
        assert_y_close(host(dn["y"]), oracle.dequant(acc, host(up["q_scale"]), g), "down y")
        log(f"[workload] batched decode M={M}: near-tie flips {flips}")


def test_workload_prefill():
    """M=4096 prefill chain, seed 3, in the launches the benchmark times
    (quantiser, up GEMM + ReLU^2 with the subln requantisation, down GEMM):
    every row of every stage against the oracle, teacher-forced (xq, scales
    and row sums, acc_up, y1, the requantised rows, acc_down, y)."""
    d = synth.prefill()
    X = d["X"]
    M = X.shape[0]
    pu, su, qu, gu = check_pack(d["W_up"], "prefill up")
    pd, sd, qd, gd = check_pack(d["W_down"], "prefill down")
    log(f"[workload] prefill M=4096 (oracle on {oracle.threads()} threads)")
    xq, xs, rs = bl.quant_act(dev(X))
    up = bl.forward(xq, xs, pu, su, x_rowsum=rs, relu2=True, subln=True, want_acc=True)
    dn = bl.forward(up["q"], up["q_scale"], pd, sd, x_rowsum=up["q_rowsum"], want_acc=True)
    torch.cuda.synchronize()
    rq = oracle.quant_act(X)
    assert_exact(host(xq), rq[0], "xq")
    assert_exact(host(xs), rq[1], "scale")
    assert_exact(host(rs), rq[2], "rowsum")
    acc = oracle.int_matmul(rq[0], qu)
    assert_exact(host(up["acc"]), acc, "up acc")
    y1 = host(up["y"])
    assert_y_close(y1, oracle.relu2(oracle.dequant(acc, rq[1], gu)), "up y")
    del acc
    flips = check_requant(oracle.rmsnorm(y1), host(up["q"]), host(up["q_scale"]), host(up["q_rowsum"]),
                          "prefill subln")
    del y1
    q2 = host(up["q"])
    acc2 = oracle.int_matmul(q2, qd)
    assert_exact(host(dn["acc"]), acc2, "down acc")
    assert_y_close(host(dn["y"]), oracle.dequant(acc2, host(up["q_scale"]), gd), "down y")
    assert np.all(np.abs(q2).max(axis=1) == 127)
    log(f"[workload] prefill: {M} rows compared at every stage, near-tie flips {flips}")


def test_attention_projections():
    """The attention block's BitLinear shapes (q, o 2560->2560; k, v
    2560->640; 2560->3840) at M = 1, 5, 130, through bitlinear_forward and,
    for M <= 4, the fused quantise + forward; every element against the
    oracle (M = 130 runs the GEMM, M <= 64 the batched kernel)."""
    d = synth.attention_projections()
    for name in ("q", "k", "v", "o", "qkv"):
        W = d[f"W_{name}"]
        p, s, q, g = check_pack(W, f"attention {name}")
        for M in (1, 5, 130):
            X = d[f"X{M}"]
            log(f"[attention] {name} N={W.shape[0]} M={M}")
            ref = oracle.bitlinear(X, q, g)
            xq, xs, rs = bl.quant_act(dev(X))
            out = bl.forward(xq, xs, p, s, x_rowsum=rs, want_acc=True)
            assert_exact(host(out["acc"]), ref["acc"], f"{name} M={M} acc")
            assert_y_close(host(out["y"]), ref["y"], f"{name} M={M} y")
            if M <= 4:
                y = bl.quant_forward(dev(X), p, s)
                assert_exact(host(y), host(out["y"]), f"{name} M={M} fused vs staged")


@pytest.mark.parametrize("M", [1, 32])
def test_workload_ffn_stack(M):
    """30-layer FFN stack, seed 4, M=1 and M=32: every row of every layer
    teacher-forced through the staged calls (each stage against the oracle),
    the stack call exactly equal to the staged calls, and, for information,
    the free-running difference from the oracle's own 30-layer chain."""
    log(f"[workload] ffn stack M={M}: generating 30 layers")
    gl, ol = [], []
    rng = None
    for rng, l, Wu, Wd in synth.ffn_stack_weights():
        g, o = to_gpu_layers([(Wu, Wd, None, None)])
        gl += g
        ol += o
    h0 = synth.ffn_stack_hidden(rng)[:M].copy()
    hs = dev(h0)
    log(f"[workload] ffn stack M={M}: running")
    stack = bl.FFNStack(gl, synth.HIDDEN, synth.FFN, M, DEV)
    stack(hs)
    got = host(hs)
    h = h0
    flips = 0
    for l in range(len(gl)):
        h, f = layer_teacher_forced(h, gl[l], ol[l], M)
        flips += f
    assert_exact(got, h, "stack call vs staged calls")
    ref = oracle.ffn_stack(h0, ol)
    rel = np.abs(got - ref).max(axis=1) / np.abs(ref).max(axis=1)
    log(f"[workload] ffn stack M={M}: {M} rows x 30 layers teacher-forced, near-tie flips {flips}; "
        f"free running after 30 layers: max |diff| / max |h| per row: max {rel.max():.3g}, median "
        f"{np.median(rel):.3g}")


# ------------------------------------------------------------------ persistent one-token stack

@pytest.mark.parametrize("H,F,L,pre,residual", [(256, 640, 3, True, True), (512, 1536, 2, False, True),
                                                 (256, 1024, 5, True, False), (1024, 256, 2, True, True)])
def test_ffn_persistent_small(H, F, L, pre, residual):
    """The one-launch persistent stack (BL_FFN_PERSISTENT) at one token gives
    bit for bit the two-launch-per-layer path's hidden state (itself checked
    stage by stage against the oracle), with gains, with and without the
    pre-norm and the residual, a hidden row longer than the intermediate one,
    on two calls in a row."""
    log(f"[persistent] H={H} F={F} L={L} pre={pre} residual={residual}")
    rng = np.random.default_rng(5100 + H + F + L)
    gl, ol = to_gpu_layers(ffn_layers_np(rng, L, H, F, gains=True))
    h0 = synth.activations(rng, 1, H, outliers=True)
    ref = dev(h0)
    bl.FFNStack(gl, H, F, 1, DEV, pre_norm=pre, residual=residual)(ref)
    stack = bl.FFNStack(gl, H, F, 1, DEV, pre_norm=pre, residual=residual, persistent=True)
    for rep in range(2):
        h = dev(h0)
        stack(h)
        assert_exact(host(h), host(ref), f"persistent vs two launches per layer (call {rep})")
    # the staged path against the oracle, layer by layer
    hs = h0
    for l in range(L):
        hs, _ = layer_teacher_forced(hs, gl[l], ol[l], 1, pre=pre, residual=residual)
    assert_exact(host(ref), hs, "two launches per layer vs staged calls")


def test_ffn_persistent_chunked():
    """More layers than one persistent launch takes (48): the stack runs as
    consecutive launches, each starting from the hidden state the previous one
    stored, bit-identical to two launches per layer, on two calls in a row."""
    log("[persistent] 50 layers (two launches)")
    rng = np.random.default_rng(5300)
    H, F, L = 256, 640, 50
    gl, _ = to_gpu_layers(ffn_layers_np(rng, L, H, F, gains=True))
    h0 = synth.activations(rng, 1, H, outliers=True)
    ref = dev(h0)
    bl.FFNStack(gl, H, F, 1, DEV)(ref)
    stack = bl.FFNStack(gl, H, F, 1, DEV, persistent=True)
    for rep in range(2):
        h = dev(h0)
        stack(h)
        assert_exact(host(h), host(ref), f"persistent 50-layer stack vs two launches per layer (call {rep})")


def test_ffn_persistent_model_stack():
    """The 30-layer stack at hidden 2560 / intermediate 6912 (seed 4) at one
    token through the persistent launch: bit-identical to the two-launch path
    (which test_workload_ffn_stack checks layer by layer against the oracle),
    and a gated layer or more than one token is refused."""
    log("[persistent] 30-layer model stack, M=1")
    gl = []
    rng = None
    for rng, l, Wu, Wd in synth.ffn_stack_weights():
        pu, su = bl.pack_weights(dev(Wu))
        pd, sd = bl.pack_weights(dev(Wd))
        gl.append({"up": pu, "up_scale": su, "down": pd, "down_scale": sd})
    h0 = synth.ffn_stack_hidden(rng)[:1].copy()
    ref = dev(h0)
    bl.FFNStack(gl, synth.HIDDEN, synth.FFN, 1, DEV)(ref)
    for rep in range(2):
        h = dev(h0)
        bl.FFNStack(gl, synth.HIDDEN, synth.FFN, 1, DEV, persistent=True)(h)
        assert_exact(host(h), host(ref), f"persistent 30-layer stack vs two launches per layer (call {rep})")
    h2 = dev(synth.ffn_stack_hidden(rng)[:2].copy())
    with pytest.raises(bl.BitLinearError) as e:
        bl.FFNStack(gl, synth.HIDDEN, synth.FFN, 2, DEV, persistent=True)(h2)
    assert e.value.status == bl.BL_ERR_UNSUPPORTED
    gated = [dict(gl[0], gate=gl[1]["up"], gate_scale=gl[1]["up_scale"])]
    with pytest.raises(bl.BitLinearError):
        bl.FFNStack(gated, synth.HIDDEN, synth.FFN, 1, DEV, persistent=True)(dev(h0))
