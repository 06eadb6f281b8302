"""Pins of the oracle's packed storage and dequantizing product.

Pages: "GPTQ: fixing errors as you go" (the 4-bit Llama layer example: the
file holds 4-bit integers and one scale per 128 weights; served for
memory-bound decode); "GPTQ, Line by Line" (the AutoGPTQ example: the int4
model is about a quarter of the fp16 size). The word layout is this build's
reading; its hand-written examples below fix it."""
import numpy as np
import pytest

import oracle


def test_pack_hand_examples():
    # 4 bits: columns 0..7 hold 1..8 -> nibbles from the lowest: 0x87654321
    c = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15]], dtype=np.int64)
    p = oracle.pack_codes(c, 4)
    assert p.dtype == np.uint32 and p.shape == (1, 2)
    assert p[0, 0] == 0x87654321 and p[0, 1] == 0xF
    # 3 bits: ten codes per word, the two top bits unused
    c3 = np.array([[7, 0, 1, 2, 3, 4, 5, 6, 7, 7, 5]], dtype=np.int64)
    p3 = oracle.pack_codes(c3, 3)
    want = sum(int(v) << (3 * i) for i, v in enumerate(c3[0, :10]))
    assert p3.shape == (1, 2) and p3[0, 0] == want and p3[0, 1] == 5 and want < (1 << 30)
    # 8 bits: four bytes, little end first
    assert oracle.pack_codes(np.array([[0x11, 0x22, 0x33, 0x44]]), 8)[0, 0] == 0x44332211
    # 2 bits: sixteen codes per word
    assert oracle.pack_codes(np.full((1, 16), 3), 2)[0, 0] == 0xFFFFFFFF


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 8])
def test_unpack_inverts_pack_and_storage_size(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(7, 301))
    p = oracle.pack_codes(codes, bits)
    assert np.array_equal(oracle.unpack_codes(p, bits, 301), codes)
    k = 32 // bits
    assert p.shape == (7, -(-301 // k))
    if bits == 4:  # a quarter of fp16's 2 bytes per weight, up to the last word
        assert p.nbytes == 7 * 4 * (-(-301 // 8))


def test_dequant_matmul_hand_example():
    # W_hat = (q - z) s per group of 2 columns; y = x W_hat^T
    codes = np.array([[0, 3, 1, 2], [2, 2, 0, 1]])
    scales = np.array([[0.5, 2.0], [1.0, 0.25]])
    zeros = np.array([[1.0, 1.0], [2.0, 0.0]])
    # row 0: (0-1)*.5, (3-1)*.5, (1-1)*2, (2-1)*2 = -0.5, 1, 0, 2
    # row 1: (2-2)*1, (2-2)*1, (0-0)*.25, (1-0)*.25 = 0, 0, 0, 0.25
    x = np.array([[1.0, 2.0, 3.0, 4.0], [-1.0, 0.0, 0.5, 2.0]])
    y = oracle.dequant_matmul(x, oracle.pack_codes(codes, 2), 2, 4, scales, zeros, 2)
    np.testing.assert_array_equal(y, [[-0.5 + 2 + 0 + 8, 1.0], [0.5 + 0 + 0 + 4, 0.5]])


def test_dequant_matches_the_quantizer_output_and_g_idx():
    """The stored form reproduces the quantizer's W_hat: plain groups through
    dequantize(), act-order groups through dequantize_gidx()."""
    rng = np.random.default_rng(4)
    W = rng.standard_normal((12, 256)) * 0.02
    r = oracle.rtn(W, 4, 128)
    p = oracle.pack_codes(r["codes"], 4)
    Wd = oracle.dequant_weights(oracle.unpack_codes(p, 4, 256), r["scales"], r["zeros"], 128)
    assert np.array_equal(Wd, oracle.dequantize(r["codes"], r["scales"], r["zeros"], 128))
    gi = rng.permutation(256) // 128
    assert np.array_equal(oracle.dequant_weights(r["codes"], r["scales"], r["zeros"], 128, gi),
                          oracle.dequantize_gidx(r["codes"], r["scales"], r["zeros"], gi))
    x = rng.standard_normal((3, 256))
    y = oracle.dequant_matmul(x, p, 4, 256, r["scales"], r["zeros"], 128)
    np.testing.assert_allclose(y, x @ Wd.T, rtol=1e-13, atol=1e-15)
    assert np.all(oracle.abs_products(x, Wd) >= np.abs(y) - 1e-15)
