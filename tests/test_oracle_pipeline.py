"""Pins of the layer-by-layer (sequential) oracle against facts that do not
come from the oracle itself: a first layer that quantizes losslessly leaves
the second layer's inputs equal to the float model's; otherwise the second
layer's inputs are the quantized first layer's outputs, checked element by
element against a brute-force sum written from the dequantization formula;
and the ReLU's zero pattern."""
import numpy as np
import pytest

import oracle
from oracle.pipeline64 import quantize_one_layer, relu_to_f16, two_layer_block


def _x(n, d, seed):
    rng = np.random.default_rng(seed)
    A = rng.standard_normal((8, d)) / np.sqrt(8)
    return (rng.standard_normal((n, 8)) @ A + 0.1 * rng.standard_normal((n, d))).astype(np.float16)


def _on_grid_weights(rows, cols, bits, g, seed):
    """Rows whose every group is exactly (q - z) s with s a power of two,
    z an integer in [0, qmax] and both q = 0 and q = qmax present: the
    min/max grid of such a group is that grid, so every weight is a grid point
    and round-to-nearest reproduces it with zero error."""
    rng = np.random.default_rng(seed)
    qmax = (1 << bits) - 1
    q = rng.integers(0, qmax + 1, size=(rows, cols))
    ng = cols // g
    s = 2.0 ** rng.integers(-9, -5, size=(rows, ng))
    z = rng.integers(0, qmax + 1, size=(rows, ng)).astype(np.float64)
    for k in range(ng):
        q[:, k * g] = 0
        q[:, k * g + 1] = qmax
    gi = np.arange(cols) // g
    return (q - z[:, gi]) * s[:, gi], q


def test_lossless_first_layer_gives_the_float_models_inputs():
    n, d, m, dout, bits, g = 640, 128, 256, 96, 4, 64
    x = _x(n, d, 1)
    W1, q1 = _on_grid_weights(m, d, bits, g, 2)
    W2 = np.random.default_rng(3).standard_normal((dout, m)) * 0.02
    r = two_layer_block(x, W1, W2, bits, g, 64, chunk=300)
    assert np.array_equal(r["first"]["codes"], q1)
    assert np.all(r["first"]["losses"] == 0.0)
    y_float = np.maximum(x.astype(np.float64) @ W1.T, 0.0).astype(np.float16)
    assert np.array_equal(r["y1"], y_float)
    alone = quantize_one_layer(W2, y_float, bits, g, 64)
    for k in ("codes", "scales", "zeros"):
        assert np.array_equal(r["second"][k], alone[k]), k
    assert np.allclose(r["second"]["H"], alone["H"], rtol=0, atol=0)


def test_second_layer_inputs_are_the_quantized_first_layers_outputs():
    n, d, m, dout, bits, g = 300, 64, 48, 40, 3, 32
    x = _x(n, d, 4)
    rng = np.random.default_rng(5)
    W1 = rng.standard_normal((m, d)) * 0.05
    W2 = rng.standard_normal((dout, m)) * 0.05
    r = two_layer_block(x, W1, W2, bits, g, 32, chunk=128)
    c, s, z = r["first"]["codes"], r["first"]["scales"], r["first"]["zeros"]
    for t in (0, 7, 128, 299):
        for o in range(m):
            v = 0.0
            for col in range(d):
                k = col // g
                v += float(x[t, col]) * ((float(c[o, col]) - z[o, k]) * s[o, k])
            want = np.float16(max(v, 0.0))
            assert r["y1"][t, o] == want, (t, o, r["y1"][t, o], want)
    # and not the float model's: the first layer's rounding reaches the inputs
    y_float = np.maximum(x.astype(np.float64) @ W1.T, 0.0).astype(np.float16)
    assert np.mean(r["y1"] != y_float) > 0.5
    # the second layer's H is built from exactly these recorded values
    H2 = oracle.hessian([r["y1"]], m)
    assert np.array_equal(r["second"]["H"], H2)


def test_relu_zero_pattern_and_fp16_rounding():
    v = np.array([-3.0, -1e-30, 0.0, 2.0 ** -26, 2.0 ** -24, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 65504.0, 7.25])
    y = relu_to_f16(v)
    assert y.dtype == np.float16
    # negatives and zero -> 0; below half the smallest subnormal (2^-24) -> 0;
    # ties go to the even mantissa: 1 + 2^-11 -> 1, 1 + 3 * 2^-11 -> 1 + 2^-9
    want = np.array([0.0, 0.0, 0.0, 0.0, 2.0 ** -24, 1.0, 1.0 + 2.0 ** -9, 65504.0, 7.25])
    assert np.array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("bits,g", [(4, 64), (8, 128)])
def test_first_layer_ignores_the_second(bits, g):
    """The first layer is quantized from the block's inputs alone: changing
    the second layer's weights changes nothing about it."""
    x = _x(256, 128, 6)
    rng = np.random.default_rng(7)
    W1 = rng.standard_normal((64, 128)) * 0.02
    a = two_layer_block(x, W1, rng.standard_normal((32, 64)), bits, g, 64)
    b = two_layer_block(x, W1, rng.standard_normal((16, 64)), bits, g, 64)
    for k in ("codes", "scales", "zeros", "losses"):
        assert np.array_equal(a["first"][k], b["first"][k])
    assert np.array_equal(a["y1"], b["y1"])
