"""fp64 reference of inference with the stored quantized weights (CPU, numpy).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg. Shares no code with the HIP path.

What the pages fix: the file holds the low-bit integers and one scale per
group of 128 weights, and nothing changes at inference time except that the
weights are read in that form ("GPTQ: fixing errors as you go", the 4-bit
Llama layer example and "What it's good and bad at": served by inference
engines, faster on memory-bound decode; "GPTQ, Line by Line", the AutoGPTQ
example: the saved int4 model is about a quarter of the fp16 size).

Readings of what the pages leave open (also in the design notes):
  * packing: each row of codes is stored along the input dimension in 32-bit
    words holding floor(32 / bits) codes each (8 at 4 bits, 10 at 3 bits,
    16 at 2 bits, 4 at 8 bits), the lowest column in the lowest bits; unused
    high bits are zero;
  * the dequantized weight is (code - zero) * scale with the fp32 scale and
    zero of the code's group, the quantizer's own outputs; with act-order the
    group of column c is g_idx[c];
  * the product is y = x W_hat^T for activations x (tokens x cols, fp16 on
    the GPU), i.e. y[t, r] = sum_c x[t, c] * W_hat[r, c].
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def codes_per_word(bits: int) -> int:
    return 32 // bits


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """rows x ceil(cols / k) uint32 words, k = floor(32 / bits); the code of
    column c sits at bits [bits*(c % k), bits*(c % k) + bits) of word c // k."""
    codes = np.asarray(codes, dtype=np.uint64)
    rows, cols = codes.shape
    k = codes_per_word(bits)
    nw = (cols + k - 1) // k
    out = np.zeros((rows, nw), dtype=np.uint64)
    for c in range(cols):
        out[:, c // k] |= (codes[:, c] & ((1 << bits) - 1)) << np.uint64(bits * (c % k))
    return out.astype(np.uint32)


def unpack_codes(packed: np.ndarray, bits: int, cols: int) -> np.ndarray:
    """Inverse of pack_codes: rows x cols integer codes."""
    packed = np.asarray(packed, dtype=np.uint64)
    k = codes_per_word(bits)
    out = np.zeros((packed.shape[0], cols), dtype=np.int64)
    for c in range(cols):
        out[:, c] = (packed[:, c // k] >> np.uint64(bits * (c % k))) & ((1 << bits) - 1)
    return out


def dequant_weights(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                    groupsize: int, g_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """W_hat[r, c] = (code - zero[r, g(c)]) * scale[r, g(c)] in fp64, with
    g(c) = g_idx[c] or c // groupsize (groupsize <= 0: one group)."""
    codes = np.asarray(codes, dtype=np.float64)
    cols = codes.shape[1]
    if g_idx is None:
        g = cols if groupsize <= 0 else groupsize
        gi = np.arange(cols) // g
    else:
        gi = np.asarray(g_idx, dtype=np.int64)
    return (codes - np.asarray(zeros, np.float64)[:, gi]) * np.asarray(scales, np.float64)[:, gi]


def dequant_matmul(x: np.ndarray, packed: np.ndarray, bits: int, cols: int,
                   scales: np.ndarray, zeros: np.ndarray, groupsize: int,
                   g_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """y = x W_hat^T in fp64 from the packed words (the definition: unpack,
    dequantize, multiply)."""
    W_hat = dequant_weights(unpack_codes(packed, bits, cols), scales, zeros, groupsize, g_idx)
    return np.asarray(x, dtype=np.float64) @ W_hat.T


def abs_products(x: np.ndarray, W_hat: np.ndarray) -> np.ndarray:
    """sum_c |x[t, c] * W_hat[r, c]| for every output: the scale of the
    rounding error of any summation order of the products."""
    return np.abs(np.asarray(x, np.float64)) @ np.abs(W_hat).T
