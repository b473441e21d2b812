"""HIP graph replays of every path the benchmark times.  Each case captures
its calls into a graph, then replays it three times with eager calls of the
same path (on other inputs, into other buffers) and device synchronisations
in between, and checks every replay bit for bit against the eager result of
the same inputs.  The library itself records no memset nodes and allocates
nothing (its scratch comes from caller workspaces; the binding's output and
workspace tensors made during a capture come from the graph's pool), and
every kernel is deterministic, so replays must be exact."""
import numpy as np
import pytest

from bit_gemm_absmax_amd import synth
from tests.parity import assert_exact, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from bit_gemm_absmax_amd import bitlinear as bl  # noqa: E402

DEV = torch.device("cuda:0")
H, F = synth.HIDDEN, synth.FFN


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def packed(rng, N, K):
    return bl.pack_weights(dev(synth.weights(rng, N, K)))


def replay_matches(name, run, outputs, other):
    """run(): the captured calls, writing `outputs` (a list of tensors).
    other(): eager calls of the same path on other inputs and buffers."""
    log(f"[graph] {name}")
    run()
    want = [host(t).copy() for t in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for t in outputs:
        t.fill_(float("nan") if t.is_floating_point() else -7)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        other()
        torch.cuda.synchronize()
        for t in outputs:
            t.fill_(float("nan") if t.is_floating_point() else -7)
        g.replay()
        torch.cuda.synchronize()
        for w, t in zip(want, outputs):
            assert_exact(host(t), w, f"{name}: replay {rep}")
    del g


def ffn_layers(rng, n, gated=False):
    out = []
    for _ in range(n):
        L = {}
        if gated:
            L["gate"], L["gate_scale"] = packed(rng, F, H)
        L["up"], L["up_scale"] = packed(rng, F, H)
        L["down"], L["down_scale"] = packed(rng, H, F)
        L["pre_norm_gain"] = dev(synth.gains(rng, H))
        L["sub_norm_gain"] = dev(synth.gains(rng, F))
        out.append(L)
    return out


@pytest.mark.parametrize("M,gated,n", [(1, False, 2), (32, False, 1), (8, True, 1), (300, False, 1)])
def test_graph_ffn_stack(M, gated, n):
    """bitnet_ffn_forward (pre-norm, residual): the decode chain at M=1, the
    batched path at 8 and 32 tokens, the GEMM path at 300."""
    rng = np.random.default_rng(9100 + M)
    stack = bl.FFNStack(ffn_layers(rng, n, gated), H, F, M, DEV)
    h0, h1 = dev(synth.activations(rng, M, H)), dev(synth.activations(rng, M, H))
    hs, ho = torch.empty_like(h0), torch.empty_like(h1)

    def run():
        hs.copy_(h0)
        stack(hs)

    def other():
        ho.copy_(h1)
        stack(ho)

    replay_matches(f"ffn stack M={M} gated={gated} layers={n}", run, [hs], other)


def test_graph_ffn_persistent():
    """The one-launch persistent stack at one token (its descriptor copy and
    counter reset are a kernel of their own, no memset): graph replays equal
    the eager call."""
    rng = np.random.default_rng(9150)
    stack = bl.FFNStack(ffn_layers(rng, 3, False), H, F, 1, DEV, persistent=True)
    h0, h1 = dev(synth.activations(rng, 1, H)), dev(synth.activations(rng, 1, H))
    hs, ho = torch.empty_like(h0), torch.empty_like(h1)

    def run():
        hs.copy_(h0)
        stack(hs)

    def other():
        ho.copy_(h1)
        stack(ho)

    replay_matches("persistent ffn stack M=1", run, [hs], other)


@pytest.mark.parametrize("M,N", [(1, 6912), (3, 2560), (1, 40008)])
def test_graph_quant_forward(M, N):
    """The fused quantise + BitLinear launch, including the persistent
    streaming launch of a tall matrix (N = 40,008)."""
    rng = np.random.default_rng(9200 + M + N)
    p, s = packed(rng, N, H)
    qf = bl.QuantForward(p, s, M, relu2=True)
    x0, x1 = dev(synth.activations(rng, M, H, outliers=True)), dev(synth.activations(rng, M, H))
    y0 = torch.empty((M, N), dtype=torch.float32, device=DEV)
    y1 = torch.empty_like(y0)
    replay_matches(f"quant forward M={M} N={N}", lambda: qf(x0, y_out=y0), [y0], lambda: qf(x1, y_out=y1))


@pytest.mark.parametrize("M", [32, 1024])
def test_graph_forward(M):
    """Activation quantiser + BitLinear from int8 rows (batched kernel at 32
    tokens, GEMM at 1024) with the subln requantisation epilogue.  The
    outputs the captured calls allocate live in the graph's pool; the graph
    copies them into buffers made before the capture, which are compared."""
    rng = np.random.default_rng(9300 + M)
    p, s = packed(rng, F, H)
    x0, x1 = dev(synth.activations(rng, M, H)), dev(synth.activations(rng, M, H))
    keys = ("y", "q", "q_scale", "q_rowsum")
    bufs = {}

    def call(x):
        xq, xs, rs = bl.quant_act(x)
        return bl.forward(xq, xs, p, s, x_rowsum=rs, relu2=True, subln=True)

    def run():
        r = call(x0)
        for k in keys:
            if k not in bufs:
                bufs[k] = torch.empty_like(r[k])
            bufs[k].copy_(r[k])

    run()
    torch.cuda.synchronize()
    replay_matches(f"forward M={M} (y, requantised rows, scales, row sums)", run, [bufs[k] for k in keys],
                   lambda: call(x1))


def test_graph_latent_forward():
    """BitLinear from latent fp32 weights: the packer's two launches (binary64
    partial sums into the workspace, then ternarise) inside the graph."""
    rng = np.random.default_rng(9400)
    W = dev(synth.weights(rng, F, H))
    x0, x1 = dev(synth.activations(rng, 1, H)), dev(synth.activations(rng, 1, H))
    y0 = torch.empty((1, F), dtype=torch.float32, device=DEV)
    y1 = torch.empty_like(y0)
    s0 = torch.empty(1, dtype=torch.float32, device=DEV)
    s1 = torch.empty_like(s0)
    replay_matches("latent forward M=1", lambda: bl.latent_forward(x0, W, relu2=True, y_out=y0, w_scale_out=s0),
                   [y0, s0], lambda: bl.latent_forward(x1, W, relu2=True, y_out=y1, w_scale_out=s1))
