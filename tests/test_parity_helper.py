"""The GPU-result comparison (tests/parity.py) on the CPU: it accepts a
second valid trajectory of the same layer and rejects planted mistakes."""
import numpy as np
import pytest

import oracle
import synth
from parity import compare_sweep


@pytest.fixture(scope="module")
def case():
    L = synth.LAYERS["attn"].scaled(rows=1024, cols=1024, n=16384)
    X = synth.activations(L.x)
    W = synth.weights(L.w)
    U, _ = oracle.hinv_upper(oracle.hessian([X], L.x.d), 0.01)
    ref = oracle.gptq(W, U, 4, 128, 128, precision="f32", tie_distance=True)
    # an equally valid result: the sweep with Hinv perturbed by 3e-6 relative
    Up = np.triu(U * (1 + 3e-6 * np.random.default_rng(0).standard_normal(U.shape)))
    alt = oracle.gptq(W, Up, 4, 128, 128, precision="f32")
    return W, U, ref, alt


def _cmp(case, codes, scales, zeros):
    W, U, ref, _ = case
    return compare_sweep(codes, scales, zeros, ref, 128, W=W, U=U, bits=4)


def test_accepts_an_equally_valid_trajectory(case):
    W, U, ref, alt = case
    rep = _cmp(case, alt["codes"], alt["scales"], alt["zeros"])
    assert rep["ok"], rep
    assert rep["rows_diverged"] >= 1 and rep["raw_max_dcode"] >= 2  # reported, not failed
    assert rep["followed_max_dcode"] == 1 and rep["violations"] == 0


def test_accepts_the_oracle_itself(case):
    W, U, ref, _ = case
    rep = _cmp(case, ref["codes"], ref["scales"].astype(np.float32), ref["zeros"])
    assert rep["ok"] and rep["same"] == 1.0 and rep["near_tie_codes"] == 0


def test_rejects_a_code_two_levels_off(case):
    W, U, ref, alt = case
    c = alt["codes"].copy()
    r, j = 5, 700
    c[r, j] = c[r, j] + 2 if c[r, j] <= 13 else c[r, j] - 2
    rep = _cmp(case, c, alt["scales"], alt["zeros"])
    assert not rep["ok"] and rep["violations"] >= 1


def test_rejects_a_one_level_change_away_from_a_tie(case):
    W, U, ref, alt = case
    td = ref["tie_distance"]
    # the decision furthest from any tie, where neither run flipped
    mask = (alt["codes"] == ref["codes"])
    r, j = np.unravel_index(np.argmax(np.where(mask, td, -1)), td.shape)
    assert td[r, j] > 0.4
    c = alt["codes"].copy()
    c[r, j] = c[r, j] + 1 if c[r, j] < 15 else c[r, j] - 1
    rep = _cmp(case, c, alt["scales"], alt["zeros"])
    assert not rep["ok"] and rep["violations"] >= 1


def test_rejects_a_wrong_scale_or_zero(case):
    W, U, ref, alt = case
    s = alt["scales"].copy()
    s[3, 5] *= 1 + 5e-5
    assert not _cmp(case, alt["codes"], s, alt["zeros"])["ok"]
    z = alt["zeros"].copy()
    z[9, 2] += 1 if z[9, 2] < 15 else -1
    rep = _cmp(case, alt["codes"], alt["scales"], z)
    assert not rep["ok"]


def test_a_near_tie_zero_point_may_be_the_first_difference():
    # one group of 3 over [-0.5, 2.5] at 2 bits: -min/s = 0.5 exactly. The
    # oracle rounds the zero to 0 (codes 0, 2, 1); zero 1 is the other
    # neighbour of that tie and shifts the group's codes to 0, 3, 2.
    W = np.array([[-0.5, 2.5, 1.0]])
    U = np.eye(3)
    ref = oracle.gptq(W, U, 2, 3, 128, precision="f32", tie_distance=True)
    rep = compare_sweep(np.array([[0, 3, 2]]), ref["scales"], np.array([[1.0]]), ref, 3,
                        W=W, U=U, bits=2, min_same=0.0)
    assert rep["ok"] and rep["rows_diverged_at_zero"] == 1 and rep["near_tie_zeros"] == 1
    bad = compare_sweep(np.array([[0, 3, 2]]), ref["scales"], np.array([[0.0]]), ref, 3,
                        W=W, U=U, bits=2, min_same=0.0)
    assert not bad["ok"]
