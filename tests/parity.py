"""Comparison of the GPU sweep's outputs with the oracle's.

Reading of the code tolerance. A GPU sweep in fp32 and the fp64 oracle agree
on a code unless the oracle's grid position w/s + z lies within the fp32
state error of a rounding tie; after such a legitimate flip the row follows
a different (equally valid) compensation trajectory, so later codes and
group statistics of that row are no longer comparable element by element.
The comparison therefore checks, per row:

  * codes up to the row's first difference are identical (by definition);
  * at the first difference the codes differ by exactly one level and the
    oracle's grid position is within `tie_tol` levels of a rounding tie;
  * every group whose statistics were taken at or before that column has
    scale within `rel_tol` and an equal zero point;

and, over the whole layer, that at least `min_same` of all codes are
identical. Rows after their first difference are covered by the layer
output-error check done by the caller.
"""
from __future__ import annotations

import numpy as np


def compare_sweep(codes, scales, zeros, ref, groupsize, tie_tol=2e-3, rel_tol=1e-5,
                  min_same=0.999):
    codes = np.asarray(codes).astype(np.int64)
    scales = np.asarray(scales, dtype=np.float64)
    zeros = np.asarray(zeros, dtype=np.float64)
    rc, rs, rz = ref["codes"], ref["scales"], ref["zeros"]
    ties = ref["tie_distance"]
    rows, cols = codes.shape
    assert rc.shape == codes.shape and rs.shape == scales.shape
    diff = codes != rc
    same = 1.0 - diff.mean() if diff.size else 1.0
    div_rows = np.nonzero(diff.any(axis=1))[0]
    first = np.full(rows, cols, dtype=np.int64)
    if div_rows.size:
        first[div_rows] = np.argmax(diff[div_rows], axis=1)
    bad_first = []
    for r in div_rows:
        j = first[r]
        if abs(codes[r, j] - rc[r, j]) != 1 or ties[r, j] > tie_tol:
            bad_first.append((int(r), int(j), int(codes[r, j]), int(rc[r, j]), float(ties[r, j])))
    g = cols if groupsize <= 0 else groupsize
    gstart = np.arange(scales.shape[1]) * g
    valid = gstart[None, :] <= first[:, None]
    rel = np.abs(scales - rs) / np.maximum(np.abs(rs), 1e-30)
    bad_scale = valid & (rel > rel_tol)
    bad_zero = valid & (zeros != rz)
    rep = dict(
        same=float(same), rows_diverged=int(div_rows.size), rows=rows,
        bad_first=bad_first[:10], n_bad_first=len(bad_first),
        n_bad_scale=int(bad_scale.sum()), n_bad_zero=int(bad_zero.sum()),
        max_rel_scale_checked=float(rel[valid].max()) if valid.any() else 0.0,
        groups_checked=int(valid.sum()),
    )
    rep["ok"] = (same >= min_same and not bad_first and rep["n_bad_scale"] == 0
                 and rep["n_bad_zero"] == 0)
    return rep


def assert_sweep_parity(codes, scales, zeros, ref, groupsize, **kw):
    rep = compare_sweep(codes, scales, zeros, ref, groupsize, **kw)
    assert rep["ok"], rep
    return rep


def h_rel_error(H_gpu, H_ref):
    H_gpu = np.asarray(H_gpu, np.float64)
    return float(np.linalg.norm(H_gpu - H_ref) / np.linalg.norm(H_ref))


# Scoring of GPU results.  These evaluate the GPU's outputs; the oracle
# module only ever receives oracle-side data.
def dequant(codes, scales, zeros, groupsize=None, g_idx=None):
    """w_hat = (code - zero) * scale, with the group of column c given by
    g_idx[c] (act-order) or c // groupsize."""
    codes = np.asarray(codes, dtype=np.float64)
    if g_idx is None:
        cols = codes.shape[1]
        g = cols if groupsize is None or groupsize <= 0 else groupsize
        g_idx = np.arange(cols) // g
    gi = np.asarray(g_idx, dtype=np.int64)
    return (codes - np.asarray(zeros, np.float64)[:, gi]) * np.asarray(scales, np.float64)[:, gi]


def output_error(W, W_hat, H):
    """||(W - W_hat) X||^2 written with H = 2 X X^T: 1/2 tr(dW H dW^T)."""
    dW = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    return 0.5 * float(np.sum((dW @ np.asarray(H, np.float64)) * dW))


def damped_objective(W, W_hat, Hd):
    """Sum over rows of 1/2 dw H_d dw^T."""
    return output_error(W, W_hat, Hd)
