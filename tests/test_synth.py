"""The seeded input generators: shapes, structure and determinism."""
import numpy as np

import synth


def test_tiny_layer_shapes_and_outliers():
    L = synth.LAYERS["tiny"]
    X = synth.activations(L.x)
    W = synth.weights(L.w)
    assert X.shape == (512, 256) and X.dtype == np.float16
    assert W.shape == (64, 256) and W.dtype == np.float32
    Xf = X.astype(np.float64)
    s = Xf.std(axis=0)
    assert np.all(s[:4] > 10 * np.median(s[4:]))          # channels 0-3 scaled x20
    assert 0.015 < W.std() < 0.025


def test_chunking_does_not_change_values():
    x = synth.X_ATTN.scaled(d=256, n=3 * synth.CHUNK + 100, rank=16)
    full = synth.activations(x, threads=4)
    parts = np.concatenate(list(synth.activation_chunks(x)))
    assert np.array_equal(full, parts)
    mid = np.concatenate(list(synth.activation_chunks(x, t_begin=5000, t_end=20000)))
    assert np.array_equal(mid, full[5000:20000])
    assert np.array_equal(full, synth.activations(x, threads=1))


def test_down_projection_sparsity_and_dead_channels():
    x = synth.X_DOWN.scaled(d=1024, n=2048)
    X = synth.activations(x)
    dead = synth.dead_channels(x)
    assert dead.size == int(0.02 * 1024)
    assert np.all(X[:, dead] == 0)
    live = np.setdiff1d(np.arange(1024), dead)
    frac = (X[:, live] == 0).mean()
    assert 0.57 < frac < 0.63
    assert np.all(X >= 0)


def test_attention_outlier_channels():
    x = synth.X_ATTN.scaled(d=1024, n=2048)
    X = synth.activations(x).astype(np.float64)
    out = synth.outlier_channels(x)
    assert out.size == 10
    s = X.std(axis=0)
    rest = np.setdiff1d(np.arange(1024), out)
    assert np.all(s[out] > 10 * np.median(s[rest]))
    assert 0.9 < np.median(s[rest]) < 1.1
