"""fp64 reference of layer-by-layer quantization of a two-layer block (CPU, numpy).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg. Shares no code with the HIP path.

What the pages fix: quantization proceeds one layer at a time. For each
layer, the calibration data is run through the model and that layer's inputs
X are recorded; H = 2 X X^T is formed from them; the layer's columns are
quantized with compensation; then the next layer follows ("GPTQ: fixing
errors as you go", "The algorithm, in words"; "GPTQ > The GPTQ Algorithm",
the procedure's first step: forward hooks record each layer's inputs as the
data flows through; "GPTQ-style round-to-nearest with Hessian weighting",
"Computing the Hessian").

Readings of what the pages leave open (also in the design notes):
  * "through the model" means the model as it stands when the layer is
    reached: layers quantized before it run with their dequantized weights,
    so a later layer's H is built from the outputs of the quantized earlier
    layers;
  * the block is two linear layers with a ReLU between them,
    h = relu(x W1_hat^T), y = h W2_hat^T (W1 is m x d, W2 is d_out x m); the
    pages fix neither a block structure nor an activation;
  * the second layer's recorded input is in the activations' dtype: the
    ReLU output is rounded to fp16 (half to even), as a half-precision model
    hands it to the next layer's hook;
  * the first layer's product uses the stored form exactly: W1_hat[r, c] =
    (code - zero) * scale with the fp32 scale and zero of the code's group
    (the dequantized-weight definition of the packed-storage oracle).
"""
from __future__ import annotations

from typing import Iterator

import numpy as np

from .gptq64 import gptq, hessian, hinv_upper
from .infer64 import dequant_weights


def _chunks(X: np.ndarray, chunk: int) -> Iterator[np.ndarray]:
    for t0 in range(0, X.shape[0], chunk):
        yield X[t0:t0 + chunk]


def quantize_one_layer(W: np.ndarray, X: np.ndarray, bits: int = 4, groupsize: int = 128,
                       blocksize: int = 128, percdamp: float = 0.01, precision: str = "f32",
                       chunk: int = 8192, tie_distance: bool = False) -> dict:
    """Record-then-quantize for one layer: H from its inputs X (tokens x
    cols, as recorded), Hinv, the column sweep. Returns the sweep's dict plus
    H and U."""
    X = np.asarray(X)
    H = hessian(_chunks(X, chunk), X.shape[1])
    U, lam = hinv_upper(H, percdamp)
    out = gptq(W, U, bits, groupsize, blocksize, precision, tie_distance=tie_distance)
    out.update(H=H, U=U, lam=lam)
    return out


def relu_to_f16(v: np.ndarray) -> np.ndarray:
    """max(v, 0) rounded to fp16 (half to even): the recorded activation."""
    return np.maximum(np.asarray(v, np.float64), 0.0).astype(np.float16)


def quantized_layer_output(x: np.ndarray, codes: np.ndarray, scales: np.ndarray,
                           zeros: np.ndarray, groupsize: int) -> np.ndarray:
    """x W_hat^T in fp64 from the layer's stored form (tokens x rows)."""
    W_hat = dequant_weights(codes, scales, zeros, groupsize)
    return np.asarray(x, np.float64) @ W_hat.T


def two_layer_block(x: np.ndarray, W1: np.ndarray, W2: np.ndarray, bits: int = 4,
                    groupsize: int = 128, blocksize: int = 128, percdamp: float = 0.01,
                    precision: str = "f32", chunk: int = 8192,
                    tie_distance: bool = False) -> dict:
    """Quantize W1 (m x d) on inputs x (tokens x d, fp16), run the block's
    first half with the quantized W1 to record the second layer's inputs
    y1 = fp16(relu(x W1_hat^T)) (tokens x m), then quantize W2 (d_out x m)
    on y1. Returns dict(first=..., second=..., y1=...)."""
    x = np.asarray(x)
    first = quantize_one_layer(W1, x, bits, groupsize, blocksize, percdamp, precision, chunk,
                               tie_distance)
    y1 = np.empty((x.shape[0], np.asarray(W1).shape[0]), dtype=np.float16)
    for t0 in range(0, x.shape[0], chunk):
        y1[t0:t0 + chunk] = relu_to_f16(quantized_layer_output(
            x[t0:t0 + chunk], first["codes"], first["scales"], first["zeros"], groupsize))
    second = quantize_one_layer(W2, y1, bits, groupsize, blocksize, percdamp, precision, chunk,
                                tie_distance)
    return dict(first=first, second=second, y1=y1)
