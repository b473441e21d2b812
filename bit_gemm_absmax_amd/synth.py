"""Seeded synthetic inputs for the BitLinear W1.58A8 workloads.

This module draws random numbers only; it holds none of the layer's
arithmetic, so both the HIP path and the CPU oracle may consume its arrays.

Shapes follow the transformers "BitNet" page, section "BitNetConfig"
(hidden_size 2560, intermediate_size 6912, num_hidden_layers 30,
num_attention_heads 20, num_key_value_heads 5) and section "Model details"
(context length 4096).  Latent weights are N(0, 0.02) (the
config's initializer_range used as a plain normal std); activations are
N(0, 1), optionally with 1% of each token's entries scaled by 20.

Recipe: ``numpy.random.default_rng(seed)`` (PCG64); every draw is float64
``standard_normal`` scaled, outliers applied in float64, then cast to float32,
in the order the functions below list them.  Outliers: for each token row,
``round(0.01*K)`` distinct positions from ``rng.choice(K, ., replace=False)``
multiplied by 20.
"""
from __future__ import annotations

import numpy as np

HIDDEN = 2560
FFN = 6912
LAYERS = 30
CONTEXT = 4096
HEADS = 20
KV_HEADS = 5
HEAD_DIM = HIDDEN // HEADS          # 128
KV_DIM = KV_HEADS * HEAD_DIM        # 640
W_STD = 0.02


def weights(rng: np.random.Generator, n: int, k: int, std: float = W_STD) -> np.ndarray:
    """Latent fp32 weight [n][k] ~ N(0, std)."""
    return (rng.standard_normal((n, k)) * std).astype(np.float32)


def to_bf16(a: np.ndarray):
    """Round fp32 values to bfloat16 (nearest, ties to even; inputs finite).
    Returns (bits, values): the uint16 bit patterns and the same numbers as
    fp32 (exact: a bfloat16 is the upper half of an fp32)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    values = (bits.astype(np.uint32) << 16).view(np.float32)
    return bits, values


def weights_bf16(rng: np.random.Generator, n: int, k: int, std: float = W_STD):
    """Latent bfloat16 weight [n][k] ~ N(0, std), as (bits, fp32 values)."""
    return to_bf16(weights(rng, n, k, std))


def activations(rng: np.random.Generator, m: int, k: int, outliers: bool = False,
                frac: float = 0.01, factor: float = 20.0) -> np.ndarray:
    """fp32 activations [m][k] ~ N(0, 1); with outliers, round(frac*k) distinct
    entries of every row are multiplied by ``factor``."""
    x = rng.standard_normal((m, k))
    if outliers:
        cnt = int(round(frac * k))
        for r in range(m):
            idx = rng.choice(k, cnt, replace=False)
            x[r, idx] *= factor
    return x.astype(np.float32)


def gains(rng: np.random.Generator, k: int, lo: float = 0.5, hi: float = 1.5) -> np.ndarray:
    """Non-trivial RMSNorm gains U(lo, hi) for unit tests (workloads use ones)."""
    return rng.uniform(lo, hi, k).astype(np.float32)


# ---- the five workloads -----------------------------------------------------

def single_bitlinear(seed: int = 0, M: int = 4, K: int = 256, N: int = 512):
    """Single BitLinear, M=4, K=256, N=512."""
    rng = np.random.default_rng(seed)
    W = weights(rng, N, K)
    X = activations(rng, M, K)
    return {"W": W, "X": X}


def decode_gemv(seed: int = 1, H: int = HIDDEN, F: int = FFN):
    """Decode at model width, M=1: up 2560->6912 and down 6912->2560."""
    rng = np.random.default_rng(seed)
    W_up = weights(rng, F, H)
    W_down = weights(rng, H, F)
    X_up = activations(rng, 1, H, outliers=True)
    X_down = activations(rng, 1, F, outliers=True)
    return {"W_up": W_up, "W_down": W_down, "X_up": X_up, "X_down": X_down}


def batched_decode(seed: int = 2, Ms=(8, 32, 64), H: int = HIDDEN, F: int = FFN):
    """One layer's BitLinear set (o, gate, up, down) and X for each M."""
    rng = np.random.default_rng(seed)
    out = {"W_o": weights(rng, H, H), "W_gate": weights(rng, F, H),
           "W_up": weights(rng, F, H), "W_down": weights(rng, H, F)}
    for m in Ms:
        out[f"X{m}"] = activations(rng, m, H, outliers=True)
    return out


def prefill(seed: int = 3, M: int = CONTEXT, H: int = HIDDEN, F: int = FFN):
    """Prefill at the maximum context: up and down weights, X [M][H], no outliers."""
    rng = np.random.default_rng(seed)
    W_up = weights(rng, F, H)
    W_down = weights(rng, H, F)
    X = activations(rng, M, H)
    return {"W_up": W_up, "W_down": W_down, "X": X}


def ffn_stack_weights(seed: int = 4, layers: int = LAYERS, H: int = HIDDEN, F: int = FFN):
    """Generator of (W_up, W_down) for each layer in order, then the caller
    draws the hidden state with :func:`ffn_stack_hidden` from the same rng.

    Yields (rng, l, W_up, W_down); the rng is shared so draws stay in order."""
    rng = np.random.default_rng(seed)
    for l in range(layers):
        W_up = weights(rng, F, H)
        W_down = weights(rng, H, F)
        yield rng, l, W_up, W_down


def ffn_stack_hidden(rng: np.random.Generator, M: int = 32, H: int = HIDDEN) -> np.ndarray:
    """Initial fp32 hidden state h0 [M][H] ~ N(0, 1); the M=1 run uses row 0."""
    return rng.standard_normal((M, H)).astype(np.float32)


def attention_projections(seed: int = 5, Ms=(1, 5, 130), H: int = HIDDEN):
    """The attention block's BitLinear layers at model width: q and o
    2560->2560, k and v 2560->640 (grouped-query attention with 5 key/value
    heads of 128), and a 2560->3840 layer of the size a fused q/k/v would
    have; then token rows X for each M (with outliers)."""
    rng = np.random.default_rng(seed)
    out = {"W_q": weights(rng, H, H), "W_k": weights(rng, KV_DIM, H), "W_v": weights(rng, KV_DIM, H),
           "W_o": weights(rng, H, H), "W_qkv": weights(rng, H + 2 * KV_DIM, H)}
    for m in Ms:
        out[f"X{m}"] = activations(rng, m, H, outliers=True)
    return out
