"""Pins of the oracle's act-order variant (columns processed in decreasing
order of H_qq) against what the pages and the mathematics fix.

Pages: "GPTQ: fixing errors as you go", "The tricks that make it fast" (the
act-order addition); "GPTQ > The GPTQ Algorithm", the note on quantization
order; "GPTQ, Line by Line", the AutoGPTQ configuration (desc_act).

The readings the oracle takes where the pages are silent (stable ties,
groups of consecutive processed columns, outputs in the original column
order) are pinned here as definitions; every other check is a closed form,
an identity with the plain path, or a brute-force solve.
"""
import itertools

import numpy as np
import pytest

import oracle
import synth


def _rand_spd(d, rng, cond=1e3):
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    ev = np.geomspace(1.0, cond, d)
    return (Q * ev) @ Q.T


def _with_diag(A, diag):
    """D A D with D chosen so the result has exactly the given diagonal
    (positive definiteness is kept)."""
    s = np.sqrt(np.asarray(diag, np.float64) / np.diag(A))
    return A * np.outer(s, s)


# ------------------------------------------------------------ the order
def test_perm_is_decreasing_diagonal_with_stable_ties():
    """Brute force over all pairs: a column goes before another iff its
    diagonal is larger, or equal with a smaller index."""
    rng = np.random.default_rng(3)
    diag = rng.integers(0, 6, size=40).astype(np.float64)  # many ties, zeros
    diag[7] = -0.0
    diag[8] = 0.0
    perm = oracle.act_order_perm(diag)
    assert sorted(perm.tolist()) == list(range(40))
    pos = np.empty(40, np.int64)
    pos[perm] = np.arange(40)
    for a, b in itertools.permutations(range(40), 2):
        before = diag[a] > diag[b] or (diag[a] == diag[b] and a < b)
        assert (pos[a] < pos[b]) == before, (a, b)


def test_perm_of_sorted_diagonal_is_identity():
    assert oracle.act_order_perm(np.linspace(5.0, 1.0, 9)).tolist() == list(range(9))
    assert oracle.act_order_perm(np.ones(6)).tolist() == list(range(6))
    assert oracle.act_order_perm(np.linspace(1.0, 5.0, 5)).tolist() == [4, 3, 2, 1, 0]


# ------------------------------------------------------------ closed forms
@pytest.mark.parametrize("g", [32, 128])
def test_diagonal_hessian_is_rtn_in_processing_order(g):
    """H diagonal: every compensation term vanishes, so each column is
    rounded on its own; the groups are runs of g processed columns. The loss
    of column c is sum_r (w - w_hat)^2 (H_cc + lambda) / 2, which fixes that
    H was carried into the processing order with W."""
    rng = np.random.default_rng(5)
    d, rows = 256, 24
    hdiag = rng.permutation(np.linspace(0.5, 20.0, d))
    H = np.diag(hdiag)
    W = rng.standard_normal((rows, d)) * 0.05
    r = oracle.gptq_act_order(W, H, 0.01, bits=4, groupsize=g)
    perm = np.argsort(-hdiag, kind="stable")
    assert np.array_equal(r["perm"], perm)
    rt = oracle.rtn(W[:, perm], bits=4, groupsize=g)
    codes = np.empty_like(rt["codes"])
    codes[:, perm] = rt["codes"]
    assert np.array_equal(r["codes"], codes)
    assert np.array_equal(r["scales"], rt["scales"])
    assert np.array_equal(r["zeros"], rt["zeros"])
    gi = np.empty(d, np.int64)
    gi[perm] = np.arange(d) // g
    assert np.array_equal(r["g_idx"], gi)
    lam = 0.01 * hdiag.mean()
    What = oracle.dequantize_gidx(r["codes"], r["scales"], r["zeros"], r["g_idx"])
    loss = 0.5 * np.sum((W - What) ** 2, axis=0) * (hdiag + lam)
    np.testing.assert_allclose(r["losses"], loss, rtol=1e-12)


def test_presorted_diagonal_equals_plain_gptq():
    """If the diagonal is already decreasing, the order is the identity and
    act-order must reproduce the plain sweep exactly."""
    rng = np.random.default_rng(7)
    d = 192
    H = _with_diag(_rand_spd(d, rng, cond=50), np.linspace(10.0, 1.0, d))
    W = rng.standard_normal((16, d)) * 0.05
    r = oracle.gptq_act_order(W, H, 0.01, bits=3, groupsize=64)
    U, _ = oracle.hinv_upper(H, 0.01)
    p = oracle.gptq(W, U, 3, 64, 128)
    assert r["perm"].tolist() == list(range(d))
    for k in ("codes", "scales", "zeros", "losses"):
        assert np.array_equal(r[k], p[k]), k
    assert np.array_equal(r["g_idx"], np.arange(d) // 64)


def test_relabelled_inputs_give_relabelled_outputs():
    """The order depends only on the diagonal values, so relabelling the
    input channels (W's columns with H's rows and columns) relabels the
    outputs and leaves scales and zeros unchanged. A perm/inverse-perm mixup
    in the un-permutation fails this."""
    rng = np.random.default_rng(11)
    d = 96
    H = _with_diag(_rand_spd(d, rng, cond=40), rng.permutation(np.linspace(1.0, 8.0, d)))
    W = rng.standard_normal((12, d)) * 0.05
    sigma = rng.permutation(d)
    a = oracle.gptq_act_order(W, H, 0.01, bits=4, groupsize=32)
    b = oracle.gptq_act_order(W[:, sigma], H[np.ix_(sigma, sigma)], 0.01, bits=4, groupsize=32)
    assert np.array_equal(b["codes"], a["codes"][:, sigma])
    np.testing.assert_allclose(b["losses"], a["losses"][sigma], rtol=1e-9, atol=1e-15)
    assert np.array_equal(b["g_idx"], a["g_idx"][sigma])
    np.testing.assert_allclose(b["scales"], a["scales"], rtol=1e-12)
    assert np.array_equal(b["zeros"], a["zeros"])
    assert np.array_equal(sigma[b["perm"]], a["perm"])


def test_act_order_compensation_matches_bruteforce_obs_solve():
    """For d <= 4, after the first q+1 columns of the processing order are
    fixed at their quantized values, the other weights must be the exact
    minimizer of 1/2 (w - w0) H_d (w - w0)^T over them:
        w_F = w0_F - H_FF^{-1} H_FP (w_hat_P - w0_P),
    with P and F in the ORIGINAL column indexing (general linear solve)."""
    rng = np.random.default_rng(13)
    for d in (2, 3, 4):
        for trial in range(5):
            H = _with_diag(_rand_spd(d, rng, cond=30), rng.permutation(np.arange(1.0, d + 1.0)))
            W = rng.standard_normal((6, d))
            r = oracle.gptq_act_order(W, H, 0.01, bits=2, groupsize=d, trace=True)
            perm = r["perm"]
            Hd = H + r["lam"] * np.eye(d)
            What = oracle.dequantize_gidx(r["codes"], r["scales"], r["zeros"], r["g_idx"])
            for q in range(d - 1):
                P = sorted(perm[:q + 1].tolist())
                F = sorted(perm[q + 1:].tolist())
                dP = What[:, P] - W[:, P]
                wF = W[:, F] - np.linalg.solve(Hd[np.ix_(F, F)], Hd[np.ix_(F, P)] @ dP.T).T
                np.testing.assert_allclose(r["trace"][q][:, F], wF, rtol=1e-10, atol=1e-12)


def test_act_order_losses_sum_to_damped_objective():
    """The per-column losses still add up to 1/2 dw H_d dw^T over the
    original columns (the objective does not depend on the order)."""
    L = synth.LAYERS["tiny"]
    X = synth.activations(L.x)
    W = synth.weights(L.w)
    H = oracle.hessian([X], L.x.d)
    r = oracle.gptq_act_order(W, H, 0.01, 4, 128)
    What = oracle.dequantize_gidx(r["codes"], r["scales"], r["zeros"], r["g_idx"])
    Hd = H + r["lam"] * np.eye(L.x.d)
    assert r["losses"].sum() == pytest.approx(oracle.layer_objective(W, What, Hd).sum(), rel=1e-10)
