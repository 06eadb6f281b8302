"""Comparison of the GPU sweep's outputs with the oracle's.

Every integer decision of the sweep rounds an unrounded value: w/s + z for a
code, -min/s for a group's zero point. A GPU sweep in fp32 and the fp64
oracle take the same decision unless that value lies within the fp32 state
error of a rounding boundary; there either neighbour is a correct outcome,
and everything after it in that row follows from the one taken. Two correct
runs therefore agree on a row up to its first near-tie flip and then drift
apart: a free column-by-column comparison of two fp64 oracle runs whose Hinv
differ by 3e-6 relative already shows later codes two or three levels apart
(pinned in tests/test_oracle.py). The comparison has two parts:

raw, against the oracle's own free sweep
  * at least `min_same` of all codes identical;
  * per row, everything up to the first difference identical (by
    definition). The first difference is a code, or the zero point of the
    group that starts there. A code differs by exactly one level with the
    oracle's grid position within `tie_tol` levels of a rounding tie; a zero
    point differs by exactly one with -min/s within `tie_tol` of a tie (the
    followed sweep's judgement, which at that point starts from the same
    state as the free one);
  * every group whose statistics were taken at or before that column: scale
    within `rel_tol`; zero point equal unless it is that first difference;
  * reported, not asserted: the largest |code difference| anywhere and how
    many codes differ by more than one level.

followed, against the oracle's sweep through the GPU's near-tie decisions
  The oracle sweeps again, taking the GPU's decision wherever it is the
  other neighbour of a near tie (oracle.gptq's ``follow``), so every later
  decision is checked from the state the GPU's row was in. Then:
  * every code and every zero point of every compared row is the oracle's own
    rounding at that state or a near-tie neighbour of it (no violations), so
    every code is within one level of the oracle's decision;
  * at least `min_same` of all codes are the oracle's own decision;
  * every scale of every group within `rel_tol` of the oracle's.
"""
from __future__ import annotations

import numpy as np

import oracle


def compare_sweep(codes, scales, zeros, ref, groupsize, *, W, U, bits, blocksize=128,
                  tie_tol=2e-3, rel_tol=1e-5, min_same=0.999):
    """`ref` is oracle.gptq(W, U, bits, groupsize, blocksize, precision="f32",
    tie_distance=True); W and U are the oracle's inputs (W in processing
    order, U in fp64)."""
    codes = np.asarray(codes).astype(np.int64)
    scales = np.asarray(scales, dtype=np.float64)
    zeros = np.asarray(zeros, dtype=np.float64)
    rc, rs, rz = ref["codes"], ref["scales"], ref["zeros"]
    ties = ref["tie_distance"]
    rows, cols = codes.shape
    assert rc.shape == codes.shape and rs.shape == scales.shape
    fol = oracle.gptq(W, U, bits, groupsize, blocksize, precision="f32", tie_tol=tie_tol,
                      follow=dict(codes=codes, zeros=zeros))

    diff = codes != rc
    same = 1.0 - diff.mean() if diff.size else 1.0
    absd = np.abs(codes - rc)
    g = cols if groupsize <= 0 else groupsize
    gstart = np.arange(scales.shape[1]) * g
    zdiff = zeros != rz
    first_code = np.where(diff.any(axis=1), np.argmax(diff, axis=1), cols)
    first_zg = np.where(zdiff.any(axis=1), np.argmax(zdiff, axis=1), scales.shape[1])
    first_zc = np.where(first_zg < scales.shape[1], gstart[np.minimum(first_zg, len(gstart) - 1)],
                        cols)
    by_zero = first_zc <= first_code
    first = np.minimum(first_code, first_zc)
    div_rows = np.nonzero(first < cols)[0]
    bad_first = []
    for r in div_rows:
        if by_zero[r]:
            k = first_zg[r]
            if abs(zeros[r, k] - rz[r, k]) != 1 or not fol["zero_alternatives"][r, k]:
                bad_first.append((int(r), int(gstart[k]), "zero", float(zeros[r, k]),
                                  float(rz[r, k])))
        else:
            j = first[r]
            if abs(codes[r, j] - rc[r, j]) != 1 or ties[r, j] > tie_tol:
                bad_first.append((int(r), int(j), "code", int(codes[r, j]), int(rc[r, j]),
                                  float(ties[r, j])))
    valid = gstart[None, :] <= first[:, None]
    rel = np.abs(scales - rs) / np.maximum(np.abs(rs), 1e-30)
    bad_scale = valid & (rel > rel_tol)
    zvalid = valid & ~((gstart[None, :] == first[:, None]) & by_zero[:, None])
    bad_zero = zvalid & zdiff
    fdiff = np.abs(codes - fol["own_codes"])
    frel = np.abs(scales - fol["scales"]) / np.maximum(np.abs(fol["scales"]), 1e-30)
    rep = dict(
        same=float(same), rows_diverged=int(div_rows.size), rows=rows,
        rows_diverged_at_zero=int(by_zero[div_rows].sum()),
        raw_max_dcode=int(absd.max()) if absd.size else 0,
        raw_codes_over_1=int((absd > 1).sum()),
        bad_first=bad_first[:10], n_bad_first=len(bad_first),
        n_bad_scale=int(bad_scale.sum()), n_bad_zero=int(bad_zero.sum()),
        max_rel_scale_checked=float(rel[valid].max()) if valid.any() else 0.0,
        groups_checked=int(valid.sum()),
        followed_same=float(1.0 - fol["alternatives"].mean()) if codes.size else 1.0,
        near_tie_codes=int(fol["alternatives"].sum()),
        near_tie_zeros=int(fol["zero_alternatives"].sum()),
        violations=int(fol["violations"].sum()),
        zero_violations=int(fol["zero_violations"].sum()),
        followed_max_dcode=int(fdiff.max()) if fdiff.size else 0,
        followed_max_rel_scale=float(frel.max()) if frel.size else 0.0,
    )
    if rep["violations"]:
        r, c = np.argwhere(fol["violations"])[0]
        rep["first_violation"] = (int(r), int(c), int(codes[r, c]), int(fol["own_codes"][r, c]))
    rep["ok"] = (same >= min_same and not bad_first and rep["n_bad_scale"] == 0
                 and rep["n_bad_zero"] == 0 and rep["violations"] == 0
                 and rep["zero_violations"] == 0 and rep["followed_max_dcode"] <= 1
                 and rep["followed_same"] >= min_same
                 and rep["followed_max_rel_scale"] <= rel_tol)
    return rep


def assert_sweep_parity(codes, scales, zeros, ref, groupsize, **kw):
    rep = compare_sweep(codes, scales, zeros, ref, groupsize, **kw)
    assert rep["ok"], rep
    return rep


def h_rel_error(H_gpu, H_ref):
    H_gpu = np.asarray(H_gpu, np.float64)
    return float(np.linalg.norm(H_gpu - H_ref) / np.linalg.norm(H_ref))


# Scoring of GPU results.
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
