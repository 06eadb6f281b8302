"""fp64 reference implementation of GPTQ on one linear layer (CPU, numpy).

TEST INFRASTRUCTURE: imported only by tests, the smoke check and the
benchmark's CPU-baseline leg. Shares no code with the HIP path.

Sources (page titles and sections):
  [GA]  "GPTQ > The GPTQ Algorithm" -- the three modifications to OBQ and
        the step-by-step procedure.
  [FE]  "GPTQ: fixing errors as you go" -- sections "The algorithm, in words",
        "The tricks that make it fast", "Objective", "The OBQ update".
  [RTN] "GPTQ-style round-to-nearest with Hessian weighting" -- the
        ``gptq_quantize_layer`` and ``collect_hessian`` listings.
  [LL]  "GPTQ, Line by Line: Hessian-Based Weight Quantization" -- the
        questions on the Hessian, percdamp, blocks of 128 and Cholesky.

Conventions. W is rows x cols (output x input features). X is given
token-major (tokens x cols), the layout a forward hook records, so the
pages' H = 2 X X^T (X feature-major) is 2 * X_tok^T X_tok here. Everything is
float64 except where ``precision="f32"`` asks for the quantizer's integer
decisions (group min/max -> scale, zero; w/s + z -> code) to be taken in IEEE
float32 arithmetic, the precision the [RTN] listing runs its quantizer in;
the compensation state stays float64 in both modes.

Readings of points the pages leave open (each also listed in the design
notes):
  * H is not divided by the token count and keeps the factor 2 ([FE]
    "Objective"); any positive rescaling leaves the codes unchanged because
    the damping is relative.
  * The damping mean is taken over the undamped diagonal, dead channels
    included ([RTN] listing, [LL] percdamp).
  * Hinv is the upper Cholesky factor U of H_d^{-1} (H_d^{-1} = U^T U); row q
    of U from q onward is the compensation direction and U[q,q] the divisor
    ([LL] Cholesky question; [GA] "Cholesky-based inverse updates" states the
    same object through its transpose).
  * The min/max range is not widened to include 0; the zero point is clamped
    to [0, 2^b - 1]; scale is floored at 1e-8; rounding is half-to-even
    ([RTN] listing).
  * Group statistics are taken when the sweep reaches a group's first
    column, from the current (compensated) weights ([RTN] listing).
  * A short last group covers the remaining columns.
  * Per-column loss is the OBS increase (w - w_hat)^2 / (2 U[q,q]^2) summed
    over rows ([FE] "The OBQ update": the cost of an error is governed by
    the diagonal of the downdated inverse).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np
from scipy.linalg import lapack, solve_triangular


class NotPositiveDefinite(ArithmeticError):
    """A Cholesky pivot was <= 0 or NaN. ``info`` is 1-based; values in
    [1, d] refer to the factorization of the damped Hessian, values in
    [d+1, 2d] to the re-factorization of its inverse."""

    def __init__(self, info: int):
        super().__init__(f"matrix not positive definite (info={info})")
        self.info = int(info)


# --------------------------------------------------------------------------
# H = 2 X X^T  ([FE] "The algorithm, in words" and "Objective"; [RTN]
# "Computing the Hessian": the hook adds x^T x batch by batch)
# --------------------------------------------------------------------------
def hessian(chunks: Iterable[np.ndarray], d: int, alpha: float = 2.0) -> np.ndarray:
    """Sum of alpha * Xc^T Xc over token-major chunks Xc (tokens x d), fp64."""
    H = np.zeros((d, d), dtype=np.float64)
    for Xc in chunks:
        Xc = np.asarray(Xc, dtype=np.float64)
        if Xc.shape[0] == 0:
            continue
        assert Xc.shape[1] == d
        H += alpha * (Xc.T @ Xc)
    return H


# --------------------------------------------------------------------------
# Damping ([LL] "What does percdamp do": add percdamp * mean(diag H) to every
# diagonal entry before factorizing; [RTN] listing does the same with 0.01)
# --------------------------------------------------------------------------
def damp(H: np.ndarray, percdamp: float):
    lam = percdamp * float(np.mean(np.diag(H)))
    Hd = np.array(H, dtype=np.float64, copy=True)
    Hd[np.diag_indices_from(Hd)] += lam
    return Hd, lam


def cholesky_lower(A: np.ndarray, info_offset: int = 0) -> np.ndarray:
    """Lower Cholesky factor L (A = L L^T). Raises NotPositiveDefinite with the
    1-based index of the first pivot that is <= 0 or NaN."""
    A = np.asarray(A, dtype=np.float64)
    if A.shape[0] == 0:
        return A.copy()
    L, info = lapack.dpotrf(A, lower=1, clean=1, overwrite_a=0)
    if info > 0:
        raise NotPositiveDefinite(info + info_offset)
    if info < 0:
        raise ValueError(f"dpotrf argument error {info}")
    if not np.all(np.isfinite(L)):
        bad = np.nonzero(~np.isfinite(np.diag(L)))[0]
        raise NotPositiveDefinite((int(bad[0]) if bad.size else 0) + 1 + info_offset)
    return L


def inverse_from_cholesky(L: np.ndarray) -> np.ndarray:
    """H^{-1} = L^{-T} L^{-1} from the lower factor, by solving against the
    identity ([LL] Cholesky question: the inverse is formed from the
    factorization, not by a general inversion)."""
    d = L.shape[0]
    Linv = solve_triangular(L, np.eye(d), lower=True)
    return Linv.T @ Linv


def hinv_upper(H: np.ndarray, percdamp: float):
    """Damp H, factor it, form its inverse, and return the upper Cholesky
    factor U of that inverse (H_d^{-1} = U^T U), plus lambda.

    [LL] Cholesky question (three steps: factor, invert through the factor,
    upper-factor the inverse); [RTN] listing (cholesky, cholesky_inverse,
    cholesky upper)."""
    d = H.shape[0]
    Hd, lam = damp(H, percdamp)
    L = cholesky_lower(Hd)
    Hi = inverse_from_cholesky(L)
    Hi = 0.5 * (Hi + Hi.T)
    U = cholesky_lower(Hi, info_offset=d).T.copy()
    return U, lam


# --------------------------------------------------------------------------
# Quantizer ([RTN] listing: asymmetric min/max grid per row and group)
# --------------------------------------------------------------------------
def group_params(G: np.ndarray, bits: int, precision: str = "f64", position: bool = False):
    """Per-row scale and zero point from the current values G (rows x g).
    With ``position`` also the unrounded zero position -min/s."""
    qmax = (1 << bits) - 1
    if precision == "f64":
        G = np.asarray(G, dtype=np.float64)
        mn, mx = G.min(axis=1), G.max(axis=1)
        s = np.maximum((mx - mn) / qmax, 1e-8)
        tz = -mn / s
    elif precision == "f32":
        G = np.asarray(G, dtype=np.float64).astype(np.float32)
        mn, mx = G.min(axis=1), G.max(axis=1)
        s = np.maximum((mx - mn) / np.float32(qmax), np.float32(1e-8))
        tz = -mn / s
    else:
        raise ValueError(precision)
    z = np.clip(np.rint(tz), 0, qmax)
    s, z, tz = s.astype(np.float64), z.astype(np.float64), tz.astype(np.float64)
    return (s, z, tz) if position else (s, z)


def _near_tie_alternative(given, own, t, tie_tol):
    """True where the integer decision `given` differs from this sweep's own
    rounding `own` of the unrounded value t by one level and t lies within
    tie_tol levels of the rounding boundary between the two: a perturbation
    of t of that size decides for either neighbour."""
    lo = np.minimum(given, own)
    return (np.abs(given - own) == 1) & (np.abs(t - (lo + 0.5)) <= tie_tol)


def grid_position(w: np.ndarray, s: np.ndarray, z: np.ndarray,
                  precision: str = "f64") -> np.ndarray:
    """t = w/s + z, the unrounded position of w on the integer grid."""
    if precision == "f64":
        return np.asarray(w, np.float64) / s + z
    if precision == "f32":
        w32 = np.asarray(w, dtype=np.float64).astype(np.float32)
        return (w32 / s.astype(np.float32) + z.astype(np.float32)).astype(np.float64)
    raise ValueError(precision)


def quantize(w: np.ndarray, s: np.ndarray, z: np.ndarray, bits: int,
             precision: str = "f64") -> np.ndarray:
    """Integer codes clamp(round(w/s + z), 0, 2^b - 1), half-to-even."""
    qmax = (1 << bits) - 1
    return np.clip(np.rint(grid_position(w, s, z, precision)), 0, qmax)


# --------------------------------------------------------------------------
# The column sweep with lazy block updates
#   [GA] "Column-wise processing" (one fixed column order shared by all rows),
#   "Lazy batch updates" (blocks of 128), the procedure's step 3;
#   [FE] "The OBQ update" (error divided by the inverse-Hessian diagonal,
#   pushed along the inverse-Hessian row);
#   [LL] blocks-of-128 question (rank-one updates inside the block, then
#   Err1 @ Hinv[block, rest] on the rest of the matrix);
#   [RTN] listing (group statistics at the group's first column).
# --------------------------------------------------------------------------
def gptq(W: np.ndarray, U: np.ndarray, bits: int = 4, groupsize: int = 128,
         blocksize: int = 128, precision: str = "f64", trace: bool = False,
         tie_distance: bool = False, follow: Optional[dict] = None,
         tie_tol: float = 2e-3):
    """Returns dict(codes, scales, zeros, losses[, trace][, tie_distance]).

    codes  rows x cols (int64 in [0, 2^bits-1])
    scales rows x ceil(cols/groupsize), zeros likewise (integer-valued)
    losses cols: sum over rows of (w - w_hat)^2 / (2 U[j,j]^2)
    trace  (optional) list of the working matrix after each column step
    tie_distance (optional) rows x cols: distance of w/s + z from the nearest
           rounding tie (k + 1/2) when the code was decided; 0 means an exact
           tie, so a small value marks a decision that a tiny perturbation of
           the inputs can flip to the neighbouring level

    follow (optional) dict(codes=rows x cols, zeros=rows x ngroups): another
           result whose integer decisions are to be checked against this
           sweep. Every decision rounds an unrounded value (w/s + z for a
           code, -min/s for a zero point); where such a value lies within
           ``tie_tol`` levels of a rounding boundary, either neighbour is a
           correct outcome under a perturbation of the inputs that small,
           and everything after it depends on which was taken. So at each
           decision the given one is taken when it equals this sweep's own
           rounding or is the other neighbour of a near tie; otherwise this
           sweep keeps its own and counts a violation. The sweep then
           continues from the decision taken, so every later decision is
           checked from the state the given result was in. Extra outputs:
             own_codes   rows x cols, this sweep's own rounding at each step
             alternatives rows x cols bool, near-tie neighbours taken
             zero_alternatives rows x ngroups bool, likewise for zero points
             violations  rows x cols bool, code decisions that were neither
             zero_violations rows x ngroups bool, likewise for zero points
           With follow, codes and zeros are the decisions taken.
    """
    W = np.asarray(W, dtype=np.float64)
    rows, cols = W.shape
    assert U.shape == (cols, cols)
    g = cols if groupsize <= 0 else groupsize
    B = max(1, blocksize)
    ngroups = (cols + g - 1) // g
    Wk = W.copy()
    codes = np.zeros((rows, cols), dtype=np.int64)
    scales = np.zeros((rows, ngroups))
    zeros = np.zeros((rows, ngroups))
    losses = np.zeros(cols)
    states = [] if trace else None
    ties = np.zeros((rows, cols)) if tie_distance else None
    if follow is not None:
        f_codes = np.asarray(follow["codes"], dtype=np.float64)
        f_zeros = np.asarray(follow["zeros"], dtype=np.float64)
        assert f_codes.shape == (rows, cols) and f_zeros.shape == (rows, ngroups)
        own_codes = np.zeros((rows, cols), dtype=np.int64)
        alts = np.zeros((rows, cols), dtype=bool)
        viol = np.zeros((rows, cols), dtype=bool)
        zalts = np.zeros((rows, ngroups), dtype=bool)
        zviol = np.zeros((rows, ngroups), dtype=bool)
    s = z = None
    for i1 in range(0, cols, B):
        i2 = min(i1 + B, cols)
        Err1 = np.zeros((rows, i2 - i1))
        for j in range(i1, i2):
            if j % g == 0:
                s, z, tz = group_params(Wk[:, j:min(j + g, cols)], bits, precision, position=True)
                if follow is not None:
                    gz = f_zeros[:, j // g]
                    ok = (gz == z) | _near_tie_alternative(gz, z, tz, tie_tol)
                    zalts[:, j // g] = ok & (gz != z)
                    zviol[:, j // g] = ~ok
                    z = np.where(ok, gz, z)
                scales[:, j // g] = s
                zeros[:, j // g] = z
            w = Wk[:, j].copy()
            t = grid_position(w, s, z, precision)
            q = np.clip(np.rint(t), 0, (1 << bits) - 1)
            if follow is not None:
                own_codes[:, j] = q.astype(np.int64)
                gq = f_codes[:, j]
                ok = (gq == q) | _near_tie_alternative(gq, q, t, tie_tol)
                alts[:, j] = ok & (gq != q)
                viol[:, j] = ~ok
                q = np.where(ok, gq, q)
            if tie_distance:
                ties[:, j] = np.abs(np.abs(t - np.floor(t)) - 0.5)
            w_hat = (q - z) * s
            dj = U[j, j]
            e = (w - w_hat) / dj
            losses[j] = np.sum((w - w_hat) ** 2) / (2.0 * dj * dj)
            Wk[:, j:i2] -= np.outer(e, U[j, j:i2])
            Err1[:, j - i1] = e
            codes[:, j] = q.astype(np.int64)
            if trace:
                states.append(Wk.copy())
        if i2 < cols:
            Wk[:, i2:] -= Err1 @ U[i1:i2, i2:]
            if trace:
                states[-1] = Wk.copy()
    out = dict(codes=codes, scales=scales, zeros=zeros, losses=losses)
    if trace:
        out["trace"] = states
    if tie_distance:
        out["tie_distance"] = ties
    if follow is not None:
        out.update(own_codes=own_codes, alternatives=alts, violations=viol,
                   zero_alternatives=zalts, zero_violations=zviol)
    return out


def rtn(W: np.ndarray, bits: int = 4, groupsize: int = 128, precision: str = "f64"):
    """Round-to-nearest with the same grid, every weight on its own
    ([FE] "What actually matters")."""
    W = np.asarray(W, dtype=np.float64)
    rows, cols = W.shape
    g = cols if groupsize <= 0 else groupsize
    ngroups = (cols + g - 1) // g
    codes = np.zeros((rows, cols), dtype=np.int64)
    scales = np.zeros((rows, ngroups))
    zeros = np.zeros((rows, ngroups))
    for k in range(ngroups):
        c0, c1 = k * g, min((k + 1) * g, cols)
        s, z = group_params(W[:, c0:c1], bits, precision)
        scales[:, k], zeros[:, k] = s, z
        for j in range(c0, c1):
            codes[:, j] = quantize(W[:, j], s, z, bits, precision).astype(np.int64)
    return dict(codes=codes, scales=scales, zeros=zeros)


def dequantize(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
               groupsize: int) -> np.ndarray:
    """W_hat = (code - zero) * scale, group by group."""
    cols = codes.shape[1]
    g = cols if groupsize <= 0 else groupsize
    gi = np.arange(cols) // g
    return (codes.astype(np.float64) - zeros[:, gi]) * scales[:, gi]


def output_error(W: np.ndarray, W_hat: np.ndarray, H: np.ndarray) -> float:
    """||(W - W_hat) X||_F^2 expressed through H = 2 X X^T: 1/2 tr(dW H dW^T)
    ([FE] "Objective")."""
    dW = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    return 0.5 * float(np.einsum("ij,jk,ik->", dW, H, dW, optimize=True))


def layer_objective(W: np.ndarray, W_hat: np.ndarray, Hd: np.ndarray) -> np.ndarray:
    """Per-row 1/2 dw H_d dw^T (the quantity the per-column losses add up to)."""
    dW = np.asarray(W, np.float64) - np.asarray(W_hat, np.float64)
    return 0.5 * np.einsum("ij,jk,ik->i", dW, Hd, dW, optimize=True)


# --------------------------------------------------------------------------
# Act-order (desc_act): columns processed in decreasing order of H_qq
#   "GPTQ: fixing errors as you go", "The tricks that make it fast" (the
#   act-order addition: largest H_qq first, while many columns remain to
#   absorb the error); "GPTQ > The GPTQ Algorithm", the note on quantization
#   order (ActOrder = decreasing Hessian diagonal); "GPTQ, Line by Line", the
#   AutoGPTQ configuration (desc_act).
# Readings of what the pages leave open (also in the design notes):
#   * ties in H_qq keep the original column order (a stable sort), so the
#     order is a function of the diagonal alone;
#   * the whole problem is carried into the processing order: W's columns
#     and H's rows and columns are permuted, then GPTQ runs unchanged;
#   * groups are runs of `groupsize` consecutive columns in processing
#     order; scales and zeros are indexed by those groups, and g_idx maps
#     each original column to its group;
#   * codes, losses (and the trace) are returned in the original column
#     order.
# --------------------------------------------------------------------------
def act_order_perm(diag) -> np.ndarray:
    """perm[k] = the original column processed k-th: decreasing diagonal,
    ties by increasing column index. The diagonal must be free of NaN."""
    h = np.asarray(diag, dtype=np.float64).ravel()
    return np.array(sorted(range(h.size), key=lambda c: (-h[c], c)), dtype=np.int64)


def gptq_act_order(W: np.ndarray, H: np.ndarray, percdamp: float = 0.01, bits: int = 4,
                   groupsize: int = 128, blocksize: int = 128, precision: str = "f64",
                   diag: Optional[np.ndarray] = None, trace: bool = False,
                   tie_distance: bool = False):
    """GPTQ with act-order. `diag` (default: diag(H)) is the sort key; pass
    the diagonal as the GPU reads it (fp32) when the order must match.

    Returns dict(codes, losses[, trace][, tie_distance]) in original column
    order, scales and zeros per processing-order group, g_idx (cols), perm,
    and U, the Hinv of the permuted problem (its row k belongs to the
    original column perm[k])."""
    W = np.asarray(W, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    rows, cols = W.shape
    perm = act_order_perm(np.diag(H) if diag is None else diag)
    U, lam = hinv_upper(H[np.ix_(perm, perm)], percdamp)
    r = gptq(W[:, perm], U, bits, groupsize, blocksize, precision, trace=trace,
             tie_distance=tie_distance)
    g = cols if groupsize <= 0 else groupsize
    codes = np.empty_like(r["codes"])
    codes[:, perm] = r["codes"]
    losses = np.empty(cols)
    losses[perm] = r["losses"]
    g_idx = np.empty(cols, dtype=np.int64)
    g_idx[perm] = np.arange(cols) // g
    out = dict(codes=codes, scales=r["scales"], zeros=r["zeros"], losses=losses,
               g_idx=g_idx, perm=perm, U=U, lam=lam)
    if trace:
        states = []
        for S in r["trace"]:
            T = np.empty_like(S)
            T[:, perm] = S
            states.append(T)
        out["trace"] = states
    if tie_distance:
        td = np.empty_like(r["tie_distance"])
        td[:, perm] = r["tie_distance"]
        out["tie_distance"] = td
    return out


def dequantize_gidx(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                    g_idx: np.ndarray) -> np.ndarray:
    """W_hat[:, c] = (code - zero[g_idx[c]]) * scale[g_idx[c]]."""
    gi = np.asarray(g_idx, dtype=np.int64)
    return (codes.astype(np.float64) - zeros[:, gi]) * scales[:, gi]
