"""Pins of ``oracle.quantize_layer``, the whole-layer composition the GPU results are judged
against: Hessian -> damping -> [act-order] -> factor of the permuted damped Hessian -> GPTQ,
plus RTN and both reconstruction errors on the same X.

Each pin fixes the composition by something other than the composition itself: a closed
form of the compensation on a two-column block (the OBS update written out with exact
rationals), reductions to RTN, an order that act-order must leave alone, brute-force sums
over tokens and outputs, and the failure damping exists to prevent.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
from test_oracle_pins import ar1_x


# ---------------------------------------------------------------------------------- closed form
# Three input channels.  Channels 0 and 1 are correlated, channel 2 is seen by its own token
# only, so H is block diagonal: H = 2 X^T X = [[4, 6, 0], [6, 12, 0], [0, 0, 18]].  Column 2 of
# every row holds the row's largest weight 0.875, so the per-row scale is 0.875 / 7 = 0.125,
# exactly, in float32 and float16, and column 2's own error is 0.
X3 = np.array([[1.0, 2.0, 0.0], [1.0, 1.0, 0.0], [0.0, 1.0, 0.0], [0.0, 0.0, 3.0]])
S = Fraction(1, 8)
DAMP = 0.5            # large, so that the damped and undamped compensations differ widely


def _rne(x: Fraction) -> int:
    f = x.numerator // x.denominator
    r = x - f
    if r != Fraction(1, 2):
        return f + (1 if r > Fraction(1, 2) else 0)
    return f if f % 2 == 0 else f + 1


def _code(x: Fraction) -> int:
    return max(-7, min(7, _rne(x / S)))


def _pair(w_first, w_second, h_off, h_second_damped):
    """Codes of two columns of a 2 x 2 block of H taken in this order ([GPTQ-P] "Hessian-Based
    Weight Update"): the first is rounded; the second, the only one left free, moves by the
    least-squares compensation of the first one's error, w2 + (H_12 / H_22) (w1 - what1)
    with H_22 damped."""
    q1 = _code(w_first)
    q2 = _code(w_second + h_off / h_second_damped * (w_first - S * q1))
    return q1, q2


def _closed_form_rows():
    H = 2 * X3.T @ X3
    h00, h01, h11, h22 = (Fraction(int(v)) for v in (H[0, 0], H[0, 1], H[1, 1], H[2, 2]))
    lam = Fraction(DAMP) * (h00 + h11 + h22) / 3
    # (w0 / s, w1 / s) per row
    rows = [(Fraction(245, 100), Fraction(132, 100)),    # no act-order: damping decides column 1
            (Fraction(26, 10), Fraction(16, 10)),        # act-order: column 1 compensates column 0
            (Fraction(29, 10), Fraction(16, 10))]        # act-order: damping decides column 0
    W = np.array([[float(a * S), float(b * S), 0.875] for a, b in rows])
    want_off, want_act = [], []
    for (a, b), w in zip(rows, W):
        w0, w1 = Fraction(w[0]), Fraction(w[1])
        q0, q1 = _pair(w0, w1, h01, h11 + lam)              # order 0, 1, 2
        want_off.append((q0, q1, 7))
        q1a, q0a = _pair(w1, w0, h01, h00 + lam)             # act-order: 2, 1, 0 (diag 18 > 12 > 4)
        want_act.append((q0a, q1a, 7))
    # the rows are chosen so that the compensation decides a code: with the undamped H (row 0,
    # row 2) or without column 1's compensation of column 0 (row 1) the code differs
    w = [tuple(Fraction(v) for v in W[r, :2]) for r in range(3)]
    assert _pair(w[0][0], w[0][1], h01, h11)[1] != want_off[0][1]
    assert _code(w[1][0]) != want_act[1][0]
    assert _pair(w[2][1], w[2][0], h01, h00)[1] != want_act[2][0]
    return W, np.array(want_off), np.array(want_act), float(lam)


@pytest.mark.parametrize("block_size", [1, 2, 128])
def test_layer_two_column_compensation_closed_form(block_size):
    W, want_off, want_act, lam = _closed_form_rows()
    off = O.quantize_layer(W, X3, bits=4, group_size=0, block_size=block_size, damp=DAMP)
    assert off["codes"].tolist() == want_off.tolist()
    assert off["scales"].astype(np.float64).ravel().tolist() == [0.125] * 3
    assert off["lambda"] == pytest.approx(lam, rel=1e-15)
    act = O.quantize_layer(W, X3, bits=4, group_size=0, block_size=block_size, damp=DAMP, act_order=True)
    assert act["perm"].tolist() == [2, 1, 0]
    assert act["codes"].tolist() == want_act.tolist()          # original column order
    assert act["g_idx"].tolist() == [0, 0, 0]


# ---------------------------------------------------------------------------------- reductions
def _orthogonal_x(rng, n, reps=2):
    """Each token sees one channel: X^T X is diagonal, with unequal entries."""
    rows = []
    for _ in range(reps):
        rows.append(np.diag(rng.uniform(0.3, 3.0, n)))
    return np.concatenate(rows)


@pytest.mark.parametrize("gs", [0, 32])
def test_layer_diagonal_hessian_is_rtn(gs):
    rng = np.random.default_rng(31)
    n, m = 96, 20
    W = rng.normal(0, 0.02, size=(m, n))
    X = _orthogonal_x(rng, n)
    res = O.quantize_layer(W, X, 4, gs, 32, 0.01)
    r = O.rtn(W, 4, gs)
    assert np.array_equal(res["codes"], r["codes"])
    assert np.array_equal(res["scales"].view(np.uint16), r["scales"].view(np.uint16))
    assert res["gptq_mse"] == res["rtn_mse"]
    # act-order on a diagonal H: no compensation, groups formed over the processed order, so the
    # result is RTN of the column-permuted matrix, put back in original order
    act = O.quantize_layer(W, X, 4, gs, 32, 0.01, act_order=True)
    p = act["perm"]
    d = np.diag(act["H"])
    assert np.all(np.diff(d[p]) <= 0) and sorted(p.tolist()) == list(range(n))
    rp = O.rtn(W[:, p], 4, gs)
    assert np.array_equal(act["codes"][:, p], rp["codes"])
    assert np.array_equal(act["scales"].view(np.uint16), rp["scales"].view(np.uint16))
    assert np.array_equal(act["What"][:, p], rp["What"])


def test_layer_sorted_diagonal_act_order_is_identity():
    rng = np.random.default_rng(32)
    n, m = 64, 16
    X = ar1_x(rng, 200, n, 0.8) * np.linspace(3.0, 0.5, n)[None, :]
    X = X[:, np.argsort(-np.sum(X * X, axis=0), kind="stable")]             # diag H descending
    W = rng.normal(0, 0.02, size=(m, n))
    off = O.quantize_layer(W, X, 4, 16, 16, 0.01)
    act = O.quantize_layer(W, X, 4, 16, 16, 0.01, act_order=True)
    assert act["perm"].tolist() == list(range(n))
    assert act["g_idx"].tolist() == [c // 16 for c in range(n)]
    for k in ("codes", "scales", "What", "U"):
        assert np.array_equal(off[k], act[k]), k
    assert off["gptq_mse"] == act["gptq_mse"] and off["rtn_mse"] == act["rtn_mse"]


# ---------------------------------------------------------------------------------- errors
def _brute_mse(X, W, codes, scales, g, g_idx=None):
    """(1 / (N m)) sum over tokens t and outputs o of (sum_c X[t, c] (W[o, c] - s[o, G(c)] code[o, c]))^2,
    every weight decoded by hand from its code and its group's scale."""
    N, n = X.shape
    m = W.shape[0]
    tot = 0.0
    for t in range(N):
        for o in range(m):
            y = 0.0
            for c in range(n):
                G = 0 if g == 0 else (int(g_idx[c]) if g_idx is not None else c // g)
                y += X[t, c] * (W[o, c] - float(scales[o, G]) * int(codes[o, c]))
            tot += y * y
    return tot / (N * m)


@pytest.mark.parametrize("act", [False, True])
def test_layer_errors_brute_force(act):
    rng = np.random.default_rng(33)
    N, n, m, g = 12, 8, 3, 4
    X = ar1_x(rng, N, n, 0.7) * np.array([0.5, 3.0, 1.0, 2.5, 0.7, 1.8, 0.9, 2.2])[None, :]
    W = rng.normal(0, 0.02, size=(m, n))
    res = O.quantize_layer(W, X, 4, g, 4, 0.01, act_order=act)
    if act:
        assert res["perm"].tolist() != list(range(n))                   # a real permutation
    assert res["gptq_mse"] == pytest.approx(_brute_mse(X, W, res["codes"], res["scales"], g, res["g_idx"]),
                                            rel=1e-12)
    r = res["rtn"]
    assert res["rtn_mse"] == pytest.approx(_brute_mse(X, W, r["codes"], r["scales"], g), rel=1e-12)
    assert res["n_tok"] == N
    Hb = np.array([[2 * sum(X[t, i] * X[t, j] for t in range(N)) for j in range(n)] for i in range(n)])
    assert np.allclose(res["H"], Hb, rtol=1e-14, atol=1e-14)
    assert res["lambda"] == pytest.approx(0.01 * np.trace(Hb) / n, rel=1e-14)


def test_layer_damping_makes_rank_deficient_inputs_factorable():
    """Fewer tokens than inputs: X^T X is singular; only the damping makes it positive definite."""
    rng = np.random.default_rng(34)
    n, m = 32, 8
    X = ar1_x(rng, 20, n, 0.5)
    W = rng.normal(0, 0.02, size=(m, n))
    res = O.quantize_layer(W, X, 4, 16, 16, 0.01)
    assert np.all(np.abs(res["codes"]) <= 7) and res["gptq_mse"] > 0
    with pytest.raises(O.NotPositiveDefinite):
        O.quantize_layer(W, X, 4, 16, 16, 0.0)


def test_layer_gptq_error_below_rtn_on_correlated_inputs():
    """GPTQ minimises the layer's output error column by column ([MQM] 2.1): on strongly
    correlated inputs its error over many rows is well below round-to-nearest's."""
    rng = np.random.default_rng(35)
    n, m = 64, 64
    X = ar1_x(rng, 512, n, 0.9)
    W = rng.normal(0, 0.02, size=(m, n))
    res = O.quantize_layer(W, X, 4, 32, 32, 0.01)
    assert res["gptq_mse"] < 0.8 * res["rtn_mse"]
