"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a value the pages print,
a closed form, an invariant, a special case that reduces to a different computation,
or brute force on tiny inputs.
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from conftest import read_golden
import oracle as O


def tril_ones(n):
    """Token t sees input channels 0..t with value 1.0: the last token's output is the plain
    sum of the weights, and the Cholesky factor of H^-1 is upper bidiagonal with
    U[j, j+1] / U[j, j] = -1, so the GPTQ update adds the whole residual of column j to
    column j+1, which is the error-carry rule of the lesson's Example 1.1."""
    return np.tril(np.ones((n, n)))


def gptq_full(W, X, bits, group_size, block_size, damp, scales_in=None, act_order=False):
    H = O.hessian(X)
    Hd, _ = O.damp_hessian(H, damp)
    perm = O.act_order_perm(Hd) if act_order else None
    Hp = Hd[np.ix_(perm, perm)] if perm is not None else Hd
    U = O.chol_inverse_upper(Hp)
    return O.gptq(W, U, bits, group_size, block_size, perm=perm, scales_in=scales_in), H, Hd, U


def ar1_x(rng, n_tok, n, rho=0.9):
    """Correlated calibration inputs: AR(1) across channels, unit variance."""
    x = np.empty((n_tok, n))
    x[:, 0] = rng.standard_normal(n_tok)
    for c in range(1, n):
        x[:, c] = rho * x[:, c - 1] + np.sqrt(1 - rho * rho) * rng.standard_normal(n_tok)
    return x


# ---------------------------------------------------------------------------------- p1
@pytest.mark.parametrize("block_size", [1, 2, 4, 128])
@pytest.mark.parametrize("damp", [0.0, 0.01])
def test_lesson17_six_weight_example(block_size, damp):
    g = read_golden("lesson17_example_1_1.txt")
    w = np.array([g["weights"]])
    x_in = np.array(g["inputs"])
    n = w.shape[1]
    X = tril_ones(n)
    assert np.array_equal(X[-1], x_in)       # last token carries the page's all-ones input
    s = np.array([[g["step"]]], dtype=np.float16)
    res, *_ = gptq_full(w, X, bits=4, group_size=0, block_size=block_size, damp=damp, scales_in=s)
    comp = res["What"][0]
    assert [round(v, 1) for v in comp] == g["compensated"]
    assert round(abs(comp @ x_in - w[0] @ x_in), 2) == g["compensated_abs_error"]
    r = O.rtn(w, bits=4, group_size=0, scales_in=s)["What"][0]
    assert [round(v, 1) for v in r] == g["nearest"]
    assert round(abs(r @ x_in - w[0] @ x_in), 2) == g["nearest_abs_error"]


def test_lesson17_two_weight_exercise():
    g = read_golden("lesson17_two_weights.txt")
    w = np.array([g["weights"]])
    x_in = np.array(g["inputs"])
    assert abs(w[0] @ x_in - g["true_output"]) < 1e-12
    for pair, key in (("pair_up_up", "pair_up_up_error"), ("pair_down_down", "pair_down_down_error"),
                      ("pair_up_down", "pair_up_down_error")):
        assert round(abs(np.array(g[pair]) @ x_in - g["true_output"]), 2) == g[key]
    s = np.array([[g["step"]]], dtype=np.float16)
    res, *_ = gptq_full(w, tril_ones(2), bits=4, group_size=0, block_size=128, damp=0.0, scales_in=s)
    assert [round(v, 1) for v in res["What"][0]] == g["carried"]
    assert round(float(res["What"][0] @ x_in), 1) == g["carried_output"]
    r = O.rtn(w, bits=4, group_size=0, scales_in=s)["What"][0]
    assert [round(v, 1) for v in r] == g["nearest"]


def test_error_carry_rule_equals_gptq_on_random_rows():
    """For X = lower-triangular ones the U-form loop is exactly the error-carry rule of the
    lesson's Example 1.1 on any row and grid step.  That rule keeps every prefix sum of the
    rounded weights at the grid point nearest the prefix sum of the weights (each step rounds
    the running sum less what is already placed, a multiple of the step), so the compensated
    weights are the differences of round(cumsum(w) / step) * step (no ties occur here)."""
    rng = np.random.default_rng(11)
    n = 12
    W = rng.normal(0, 0.3, size=(40, n))
    s = np.full((40, 1), 0.0625, dtype=np.float16)     # power-of-two grid: all values exact
    res, *_ = gptq_full(W, tril_ones(n), bits=8, group_size=0, block_size=5, damp=0.0, scales_in=s)
    step = float(s[0, 0])
    placed = np.rint(np.cumsum(W, axis=1) / step) * step
    comp = np.diff(np.concatenate([np.zeros((W.shape[0], 1)), placed], axis=1), axis=1)
    assert np.array_equal(res["What"], comp)


# ---------------------------------------------------------------------------------- p2 / p13 / R7 / R8
def test_levels_and_code_range():
    g = read_golden("gpt2_re_levels.txt")
    assert 2 * O.qmax(int(g["bits"])) + 1 == g["levels"]
    rng = np.random.default_rng(2)
    W = rng.normal(0, 0.02, size=(64, 512)).astype(np.float32)
    for gs in (0, 128):
        r = O.rtn(W, bits=4, group_size=gs)
        c = r["codes"]
        assert c.min() >= -7 and c.max() <= 7
        assert len(np.unique(c)) <= g["levels"]
        glen = 512 if gs == 0 else gs
        for G in range(512 // glen):
            blk = np.abs(W[:, G * glen:(G + 1) * glen].astype(np.float64))
            idx = np.argmax(blk, axis=1)
            assert np.all(np.abs(c[np.arange(64), G * glen + idx]) == 7)   # absmax element -> +-7
    assert len(np.unique(O.rtn(W, 4, 0)["codes"])) == 15


def test_rtn_ties_to_even_closed_form():
    # absmax 7 -> s = 7/7 = 1 exactly; x.5 quotients are exact ties, decided to even
    W = np.array([[7.0, -3.5, 0.5, 2.5, -1.5, 0.0, 1.0, -7.0]], dtype=np.float32)
    assert O.rtn(W, 4, 0)["codes"].tolist() == [[7, -4, 0, 2, -2, 0, 1, -7]]
    r = O.rtn(W, 4, 4)
    assert r["scales"].astype(np.float64).tolist() == [[1.0, 1.0]]
    assert r["codes"].tolist() == [[7, -4, 0, 2, -2, 0, 1, -7]]
    # absmax 3.5 -> s = 0.5; 1.25 / 0.5 = 2.5 -> 2, 0.75 / 0.5 = 1.5 -> 2
    W2 = np.array([[3.5, 1.25, 0.75, -0.25]], dtype=np.float32)
    r2 = O.rtn(W2, 4, 0)
    assert float(r2["scales"][0, 0]) == 0.5
    assert r2["codes"].tolist() == [[7, 2, 2, 0]]
    # all-zero group: s = 0, codes 0
    W3 = np.zeros((1, 8), dtype=np.float32)
    r3 = O.rtn(W3, 4, 4)
    assert r3["scales"].tolist() == [[0.0, 0.0]] and not r3["codes"].any()


def _rne_to_precision(x: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Nearest value with ``mant_bits`` significant bits (ties to even), exponent >= emin."""
    if x == 0:
        return Fraction(0)
    sgn = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits + 1)
    k = a / ulp
    f = k.numerator // k.denominator
    rem = k - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return sgn * f * ulp


def test_scale_is_one_fp32_division_then_fp16():
    rng = np.random.default_rng(3)
    absmax = np.abs(rng.normal(0, 0.05, size=400)).astype(np.float32)
    s = O.group_scales_from_absmax(absmax, 4)
    for a, got in zip(absmax, s):
        q32 = _rne_to_precision(Fraction(float(a)) / 7, 24, -126)
        want = _rne_to_precision(q32, 11, -14)
        assert Fraction(float(got)) == want


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 40), st.integers(1, 40), st.sampled_from([0, 4, 8]), st.integers(0, 2**31 - 1))
def test_rtn_error_bound_and_pack_round_trip(m, half_n, gs, seed):
    n = 2 * half_n
    if gs and n % gs:
        n = gs * max(1, n // gs)
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(3, size=(m, n)) * 0.02).astype(np.float32)
    r = O.rtn(W, 4, gs)
    s = r["scales"].astype(np.float64)
    gi = np.zeros(n, int) if gs == 0 else np.arange(n) // gs
    err = np.abs(W.astype(np.float64) - r["What"])
    assert np.all(err <= s[:, gi] / 2)                                 # never clamped for RTN
    assert np.array_equal(O.unpack_int4(O.pack_int4(r["codes"]), n), r["codes"])


# ---------------------------------------------------------------------------------- p3
@pytest.mark.parametrize("gs", [0, 128])
def test_diagonal_hessian_gptq_equals_rtn(gs):
    rng = np.random.default_rng(4)
    n, m = 256, 48
    W = rng.normal(0, 0.02, size=(m, n)).astype(np.float32)
    X = np.diag(rng.uniform(0.5, 3.0, size=n))          # one token per channel: H diagonal
    res, H, Hd, U = gptq_full(W, X, 4, gs, 128, 0.01)
    assert np.count_nonzero(U - np.diag(np.diag(U))) == 0
    r = O.rtn(W, 4, gs)
    assert np.array_equal(res["codes"], r["codes"])
    assert np.array_equal(res["scales"].view(np.uint16), r["scales"].view(np.uint16))


# ---------------------------------------------------------------------------------- p4 / R11
def test_recon_mse_trace_identity():
    rng = np.random.default_rng(5)
    X = rng.standard_normal((300, 64))
    W = rng.normal(0, 0.02, size=(40, 64))
    r = O.rtn(W, 4, 16)
    direct = O.recon_mse([X[:128], X[128:]], W, r["What"])
    H = O.hessian(X)
    assert abs(direct - O.recon_mse_trace(H, 300, W, r["What"])) <= 1e-12 * direct
    # brute force over every token and output on a tiny case
    Xs, Ws, Wh = X[:5, :6], W[:3, :6], r["What"][:3, :6]
    tot = 0.0
    for t in range(5):
        for o in range(3):
            y = sum(Xs[t, c] * (Ws[o, c] - Wh[o, c]) for c in range(6))
            tot += y * y
    assert abs(O.recon_mse(Xs, Ws, Wh) - tot / 15) <= 1e-14 * max(tot, 1e-300)


# ---------------------------------------------------------------------------------- p5
def test_storage_bits_per_weight():
    g = read_golden("gptq_page_storage.txt")
    gs = int(g["group_size"])
    m, n = 64, 4 * gs
    bits = O.storage_bytes(m, n, gs) * 8 / (m * n)
    assert bits == g["bits_per_weight_symmetric"]
    assert bits + 16 / gs == g["bits_per_weight_with_zero_point"]
    codes = O.rtn(np.random.default_rng(6).normal(size=(m, n)), 4, gs)["codes"]
    assert O.pack_int4(codes).nbytes == m * n // 2
    assert O.storage_bytes(m, n, 0) * 8 / (m * n) == 4 + 16 / n


def test_pack_layout_closed_form():
    # nibble = code + 8, even column in the low nibble
    codes = np.array([[-7, 7, 0, 1, -8 + 8, 3]], dtype=np.int8)
    assert O.pack_int4(codes).tolist() == [[0xF1, 0x98, 0xB8]]


# ---------------------------------------------------------------------------------- p6 brute force
def _brute_force_min(w, s, Hq, bits):
    """min over every code vector in [-qmax, qmax]^n of (s c - w)^T Hq (s c - w)."""
    qm = O.qmax(bits)
    n = w.size
    levels = np.arange(-qm, qm + 1, dtype=np.float64)
    L = np.linalg.cholesky(Hq + 0 * np.eye(n))
    head = max(0, n - 6)
    tail = np.array(list(itertools.product(levels, repeat=n - head)))       # (7^6, n-head)
    best = np.inf
    for pre in itertools.product(levels, repeat=head):
        C = np.concatenate([np.broadcast_to(np.array(pre), (tail.shape[0], head)), tail], axis=1)
        D = s * C - w
        e = np.sum((D @ L) ** 2, axis=1)
        best = min(best, float(e.min()))
    return best


def _row_err(w, what, Hq):
    d = what - w
    return float(d @ Hq @ d)


@pytest.mark.parametrize("n,rows", [(6, 120), (8, 8)])
def test_brute_force_optimum_bounds_gptq_and_rtn(n, rows):
    rng = np.random.default_rng(7 + n)
    bits = 3
    X = ar1_x(rng, 64, n)
    W = rng.normal(0, 0.02, size=(rows, n))
    res, H, Hd, U = gptq_full(W, X, bits, 0, 128, 0.01)
    r = O.rtn(W, bits, 0)
    assert np.array_equal(res["scales"], r["scales"])                 # same per-row scale for all three
    Hq = 0.5 * H                                                      # X^T X: the layer objective
    e_g, e_r = [], []
    for i in range(rows):
        s = float(r["scales"][i, 0])
        opt = _brute_force_min(W[i], s, Hq, bits)
        eg, er = _row_err(W[i], res["What"][i], Hq), _row_err(W[i], r["What"][i], Hq)
        assert opt <= eg * (1 + 1e-12) and opt <= er * (1 + 1e-12)
        e_g.append(eg)
        e_r.append(er)
    assert np.mean(e_g) < np.mean(e_r)


# ---------------------------------------------------------------------------------- p7 (R1)
def test_u_form_loop_equals_direct_obs():
    rng = np.random.default_rng(8)
    n, rows = 8, 400
    X = ar1_x(rng, 64, n)
    W = rng.normal(0, 0.02, size=(rows, n))
    res, H, Hd, U = gptq_full(W, X, 3, 0, 128, 0.01)
    ref = O.direct_obs(W, Hd, 3, 0)
    assert np.array_equal(res["codes"], ref["codes"])


def test_u_form_loop_equals_direct_obs_groups():
    rng = np.random.default_rng(9)
    n, rows = 12, 200
    X = ar1_x(rng, 80, n, 0.8)
    W = rng.normal(0, 0.02, size=(rows, n))
    res, H, Hd, U = gptq_full(W, X, 4, 4, 5, 0.01)
    ref = O.direct_obs(W, Hd, 4, 4)
    assert np.array_equal(res["codes"], ref["codes"])
    assert np.array_equal(res["scales"], ref["scales"])


# ---------------------------------------------------------------------------------- p8
@pytest.mark.parametrize("gs", [0, 8, 16])
def test_block_size_invariance(gs):
    rng = np.random.default_rng(10)
    n, m = 48, 64
    X = ar1_x(rng, 200, n, 0.7)
    W = rng.normal(0, 0.02, size=(m, n))
    H = O.hessian(X)
    Hd, _ = O.damp_hessian(H, 0.01)
    U = O.chol_inverse_upper(Hd)
    ref = O.gptq_unblocked(W, U, 4, gs)
    for B in (1, 3, 5, 16, 128, n):
        got = O.gptq(W, U, 4, gs, B)
        assert np.array_equal(got["codes"], ref["codes"]), B
        assert np.array_equal(got["scales"], ref["scales"]), B


# ---------------------------------------------------------------------------------- p9
def test_chol_inverse_upper_properties_and_reverse_route():
    from scipy.linalg import solve_triangular
    rng = np.random.default_rng(12)
    n = 40
    X = ar1_x(rng, 120, n, 0.6)
    X[:, 3] *= 20
    Hd, _ = O.damp_hessian(O.hessian(X), 0.01)
    U = O.chol_inverse_upper(Hd)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    assert np.max(np.abs(U.T @ U @ Hd - np.eye(n))) < 1e-10
    # reverse-order route: H = Ut Ut^T with Ut upper (Cholesky of the index-reversed matrix),
    # then U = Ut^-1 by a triangular solve
    Lr = np.linalg.cholesky(Hd[::-1, ::-1])
    Ut = Lr[::-1, ::-1]
    assert np.all(np.tril(Ut, -1) == 0)
    U2 = solve_triangular(Ut, np.eye(n), lower=False)
    assert np.max(np.abs(U2 - U)) <= 1e-11 * np.max(np.abs(U))


def test_not_positive_definite_pivot():
    with pytest.raises(O.NotPositiveDefinite) as e:
        O.chol_inverse_upper(np.zeros((5, 5)))
    assert e.value.pivot == 4
    with pytest.raises(O.NotPositiveDefinite) as e:
        O.chol_inverse_upper(np.diag([1.0, 1.0, -1.0, 1.0]))
    assert e.value.pivot == 2
    Hd, lam = O.damp_hessian(np.zeros((4, 4)), 0.01)
    assert lam == 0.0
    with pytest.raises(O.NotPositiveDefinite):
        O.chol_inverse_upper(Hd)


# ---------------------------------------------------------------------------------- p10 / R3 / R4
def test_hessian_brute_force_and_trace():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((5, 3))
    H = O.hessian([X[:2], X[2:]])
    for i in range(3):
        for j in range(3):
            assert abs(H[i, j] - 2 * sum(X[t, i] * X[t, j] for t in range(5))) < 1e-13
    Xb = rng.standard_normal((500, 30))
    Hb = O.hessian(Xb)
    assert np.array_equal(Hb, Hb.T)
    assert abs(np.trace(Hb) - 2 * np.sum(Xb * Xb)) < 1e-10 * np.trace(Hb)


def test_damping_closed_form():
    H = np.diag([1.0, 2.0, 3.0])
    H[0, 2] = H[2, 0] = 0.5
    Hd, lam = O.damp_hessian(H, 0.01)
    assert lam == pytest.approx(0.02, abs=1e-15)
    assert np.allclose(Hd, H + 0.02 * np.eye(3), atol=1e-15, rtol=0)


# ---------------------------------------------------------------------------------- p11
def test_hessian_scale_invariance_bit_exact():
    rng = np.random.default_rng(14)
    n, m = 64, 32
    X = ar1_x(rng, 256, n, 0.8)
    W = rng.normal(0, 0.02, size=(m, n))
    a, *_ = gptq_full(W, X, 4, 16, 16, 0.01)
    b, *_ = gptq_full(W, 2 * X, 4, 16, 16, 0.01)          # H -> 4 H
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["scales"], b["scales"])


# ---------------------------------------------------------------------------------- p12 / R9
def test_act_order_perm_closed_form():
    H = np.diag([3.0, 5.0, 5.0, 1.0])
    assert O.act_order_perm(H).tolist() == [1, 2, 0, 3]


def test_act_order_identity_when_sorted_and_g_idx_round_trip():
    rng = np.random.default_rng(15)
    n, m = 64, 24
    X = ar1_x(rng, 300, n, 0.5)
    X = X[:, np.argsort(-np.sum(X * X, axis=0), kind="stable")]    # diag H already descending
    W = rng.normal(0, 0.02, size=(m, n))
    a, *_ = gptq_full(W, X, 4, 16, 16, 0.01, act_order=False)
    b, H, Hd, U = gptq_full(W, X, 4, 16, 16, 0.01, act_order=True)
    assert O.act_order_perm(Hd).tolist() == list(range(n))
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])
    assert b["g_idx"].tolist() == [c // 16 for c in range(n)]
    # a real permutation: g_idx maps each original column to the group it was processed in
    X2 = ar1_x(rng, 300, n, 0.5) * rng.uniform(0.5, 3, n)[None, :]
    c, H2, Hd2, U2 = gptq_full(W, X2, 4, 16, 16, 0.01, act_order=True)
    perm = O.act_order_perm(Hd2)
    pos = np.empty(n, int)
    pos[perm] = np.arange(n)
    assert np.array_equal(c["g_idx"], pos // 16)
    Wh = O.dequant(c["codes"], c["scales"], 16, g_idx=c["g_idx"])
    assert np.array_equal(Wh, c["What"])
    assert np.array_equal(Wh[:, perm], O.dequant(c["codes"][:, perm], c["scales"], 16))


# ---------------------------------------------------------------------------------- dequant rounding
def test_dequant_rounds_once():
    s = np.array([[0.0999755859375]], dtype=np.float16)     # fp16(0.1)
    codes = np.array([[3, -7, 5, 0]], dtype=np.int8)
    out16 = O.dequant(codes, s, 0, out_dtype=np.float16)
    exact = [Fraction(float(s[0, 0])) * int(c) for c in codes[0]]
    for got, ex in zip(out16[0], exact):
        assert Fraction(float(got)) == _rne_to_precision(ex, 11, -14)
    out32 = O.dequant(codes, s, 0, out_dtype=np.float32)
    assert [Fraction(float(v)) for v in out32[0]] == exact


# ---------------------------------------------------------------------------------- f1: zero-points
# [MQM] "Affine Quantization" / "Group-wise Quantization": code = round(w / S) + Z and
# w ~ S (code - Z), one (S, Z) per row and group; [GPTQ-P] "Group Quantization": a 16-bit
# zero per group beside the 16-bit scale.

def _asym_closed_form(lo, hi, bits=4):
    """Scale and zero in exact rational arithmetic: S = fp16(fp32(fp32(hi - lo) / top)),
    Z = nearest integer to -lo / S (ties to even), clamped to [0, top]."""
    top = (1 << bits) - 1
    span = _rne_to_precision(Fraction(float(np.float32(hi))) - Fraction(float(np.float32(lo))), 24, -126)
    s = _rne_to_precision(_rne_to_precision(span / top, 24, -126), 11, -14)
    if s == 0:
        return s, 0
    q = -Fraction(float(np.float32(lo))) / s
    f = q.numerator // q.denominator
    rem = q - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return s, min(max(f, 0), top)


def test_asym_worked_group():
    # range [-1, 2]: S = fp16(3 / 15) = 0.199951171875; -lo / S = 5.0012.. -> Z = 5;
    # -1 / S = -5.0012 -> -5 + 5 = 0; -0.5 / S = -2.5006 -> -3 + 5 = 2; 0 -> 5;
    # 2 / S = 10.0024 -> 10 + 5 = 15.
    W = np.array([[-1.0, -0.5, 0.0, 2.0]], dtype=np.float32)
    r = O.rtn(W, 4, 4, sym=False)
    assert float(r["scales"][0, 0]) == 0.199951171875
    assert r["zeros"].tolist() == [[5]]
    assert r["codes"].tolist() == [[0, 2, 5, 15]]
    assert r["What"][0, 2] == 0.0
    # range [-7.5, 7.5]: S = 1 exactly, -lo / S = 7.5 is a tie -> Z = 8 (even);
    # 0.5 -> 0 + 8; -7.5 -> -8 + 8 = 0; 7.5 -> 8 + 8 = 16, clamped to 15; 2.5 -> 2 + 8
    W2 = np.array([[-7.5, 7.5, 0.5, 2.5]], dtype=np.float32)
    r2 = O.rtn(W2, 4, 0, sym=False)
    assert float(r2["scales"][0, 0]) == 1.0 and r2["zeros"].tolist() == [[8]]
    assert r2["codes"].tolist() == [[0, 15, 8, 10]]
    # one-signed groups: lo = 0 gives Z = 0; hi = 0 gives Z = top; an all-zero group S = 0
    W3 = np.array([[0.0, 1.5, 3.0, 0.1, -3.0, -1.5, 0.0, -0.1, 0, 0, 0, 0]], dtype=np.float32)
    r3 = O.rtn(W3, 4, 4, sym=False)
    assert r3["zeros"].tolist() == [[0, 15, 0]]
    assert float(r3["scales"][0, 2]) == 0.0 and not r3["codes"][0, 8:].any()
    # S = fp16(0.2) = 0.199951171875 for both: 1.5 / S = 7.5018 -> 8, 0.1 / S = 0.50012 -> 1;
    # -3 / S = -15.004 -> -15 + 15 = 0, -1.5 / S -> -8 + 15 = 7, -0.1 / S -> -1 + 15 = 14
    assert r3["codes"][0, :4].tolist() == [0, 8, 15, 1]
    assert r3["codes"][0, 4:8].tolist() == [0, 7, 15, 14]


def test_asym_scale_zero_closed_form():
    rng = np.random.default_rng(30)
    lo = np.minimum(rng.normal(0, 0.05, size=300), 0).astype(np.float32)
    hi = np.maximum(rng.normal(0, 0.05, size=300), 0).astype(np.float32)
    lo[:5] = 0.0
    hi[5:10] = 0.0
    lo[10], hi[10] = 0.0, 0.0
    for bits in (2, 3, 4, 8):
        s, z = O.asym_scale_zero(lo, hi, bits)
        for i in range(300):
            ws, wz = _asym_closed_form(float(lo[i]), float(hi[i]), bits)
            assert Fraction(float(s[i])) == ws and int(z[i]) == wz


@settings(max_examples=60, deadline=None)
@given(st.integers(1, 30), st.integers(1, 30), st.sampled_from([0, 4, 8]), st.sampled_from([2, 3, 4]),
       st.integers(0, 2**31 - 1))
def test_asym_nearest_level_bound_and_pack(m, half_n, gs, bits, seed):
    """Every code is a nearest one of the group's 2^b levels S (q - Z), q = 0 .. top (brute
    force); real 0 is a level, so a 0 weight comes back exactly; an unclamped weight is
    within S / 2; the codes survive unsigned packing."""
    n = 2 * half_n
    if gs and n % gs:
        n = gs * max(1, n // gs)
    rng = np.random.default_rng(seed)
    W = (rng.standard_t(3, size=(m, n)) * 0.02 + rng.normal(0, 0.01, size=(m, 1))).astype(np.float32)
    W[rng.random((m, n)) < 0.05] = 0.0
    r = O.rtn(W, bits, gs, sym=False)
    top = (1 << bits) - 1
    gi = np.zeros(n, int) if gs == 0 else np.arange(n) // gs
    s = r["scales"].astype(np.float64)[:, gi]
    z = r["zeros"].astype(np.float64)[:, gi]
    w = W.astype(np.float64)
    levels = s[..., None] * (np.arange(top + 1)[None, None, :] - z[..., None])
    dist = np.abs(w[..., None] - levels)
    got = np.take_along_axis(dist, r["codes"].astype(np.int64)[..., None], axis=2)[..., 0]
    assert np.all(got <= dist.min(axis=2))
    assert np.all(r["What"][W == 0] == 0)
    inner = (r["codes"] > 0) & (r["codes"] < top)
    assert np.all(np.abs(w - r["What"])[inner] <= s[inner] / 2)
    assert np.all(np.abs(w - r["What"]) <= s * (0.5 + 2.0 ** -7))
    if bits == 4:
        assert np.array_equal(O.unpack_uint4(O.pack_uint4(r["codes"]), n), r["codes"])


def test_asym_pack_layout_and_storage():
    codes = np.array([[0, 15, 5, 10, 1, 8]], dtype=np.uint8)
    assert O.pack_uint4(codes).tolist() == [[0xF0, 0xA5, 0x81]]       # nibble = code, even low
    g = read_golden("gptq_page_storage.txt")
    gs = int(g["group_size"])
    m, n = 32, 4 * gs
    assert O.storage_bytes(m, n, gs, zero_point=True) * 8 / (m * n) == g["bits_per_weight_with_zero_point"]


@pytest.mark.parametrize("gs", [0, 128])
def test_asym_diagonal_hessian_gptq_equals_rtn(gs):
    rng = np.random.default_rng(31)
    n, m = 256, 48
    W = (rng.normal(0, 0.02, size=(m, n)) + 0.01).astype(np.float32)
    X = np.diag(rng.uniform(0.5, 3.0, size=n))
    Hd, _ = O.damp_hessian(O.hessian(X), 0.01)
    res = O.gptq(W, O.chol_inverse_upper(Hd), 4, gs, 128, sym=False)
    r = O.rtn(W, 4, gs, sym=False)
    assert np.array_equal(res["codes"], r["codes"])
    assert np.array_equal(res["zeros"], r["zeros"])
    assert np.array_equal(res["scales"].view(np.uint16), r["scales"].view(np.uint16))


@pytest.mark.parametrize("gs", [0, 8])
def test_asym_u_form_loop_equals_direct_obs(gs):
    """The factor form with zero-points against sequential OBS solves (no factor at all)."""
    rng = np.random.default_rng(32)
    n, m = 24, 60
    X = ar1_x(rng, 96, n, 0.8)
    W = rng.normal(0.005, 0.02, size=(m, n))
    Hd, _ = O.damp_hessian(O.hessian(X), 0.01)
    ref = O.direct_obs(W, Hd, 4, gs, sym=False)
    U = O.chol_inverse_upper(Hd)
    for B in (1, 5, 128):
        res = O.gptq(W, U, 4, gs, B, sym=False)
        assert np.array_equal(res["codes"], ref["codes"])
        assert np.array_equal(res["zeros"], ref["zeros"])
        assert np.allclose(res["scales"].astype(np.float64), ref["scales"].astype(np.float64), rtol=0, atol=0)
    un = O.gptq_unblocked(W, U, 4, gs, sym=False)
    assert np.array_equal(un["codes"], ref["codes"])


# ---------------------------------------------------------------------------------- f2: Y = X What^T
def test_quantized_matmul_brute_force_and_identity():
    rng = np.random.default_rng(70)
    m, n, T, g = 5, 16, 3, 8
    W = rng.normal(0, 0.02, size=(m, n))
    for sym in (True, False):
        r = O.rtn(W, 4, g, sym=sym)
        X = rng.standard_normal((T, n)).astype(np.float16).astype(np.float64)
        Y = O.quantized_matmul(X, r["codes"], r["scales"], g, zeros=r["zeros"])
        # brute force: every output as a plain sum of x * s * (code - z), s and z looked up by hand
        for t in range(T):
            for o in range(m):
                tot = 0.0
                for c in range(n):
                    s = float(r["scales"][o, c // g])
                    z = 0.0 if sym else float(r["zeros"][o, c // g])
                    tot += X[t, c] * s * (float(r["codes"][o, c]) - z)
                assert abs(Y[t, o] - tot) <= 1e-15 * max(1.0, abs(tot))
        # X = I gives What^T exactly
        assert np.array_equal(O.quantized_matmul(np.eye(n), r["codes"], r["scales"], g, zeros=r["zeros"]), r["What"].T)


# ---------------------------------------------------------------------------------- f4: per tensor
def test_tensor_scales_closed_form_and_reductions():
    rng = np.random.default_rng(90)
    W = rng.normal(0, 0.02, size=(48, 256)).astype(np.float32)
    W[7, 100] = 0.3                                         # the tensor's absmax
    s, z = O.tensor_scales(W, 4)
    assert z is None and s.shape == (48, 1) and np.all(s == s[0, 0])
    q32 = _rne_to_precision(Fraction(float(np.float32(0.3))) / 7, 24, -126)
    assert Fraction(float(s[0, 0])) == _rne_to_precision(q32, 11, -14)
    r = O.rtn(W, 4, 0, scales_in=s)
    assert r["codes"][7, 100] == 7 and np.abs(r["codes"]).max() == 7
    # the tensor's absmax sets the scale, so no weight is clamped: every error is within s / 2
    err_t = np.abs(W - r["What"]).max(axis=1)
    assert np.all(err_t <= float(s[0, 0]) / 2 + 1e-12)
    # zero-point form: the flattened range, exact rationals
    s2, z2 = O.tensor_scales(W, 4, sym=False)
    ws, wz = _asym_closed_form(float(W.min()), float(W.max()), 4)
    assert Fraction(float(s2[0, 0])) == ws and int(z2[0, 0]) == wz and np.all(z2 == z2[0, 0])
    # GPTQ with a diagonal H and the tensor's scales equals RTN with them
    Hd, _ = O.damp_hessian(O.hessian(np.diag(rng.uniform(0.5, 3.0, 256))), 0.01)
    g = O.gptq(W, O.chol_inverse_upper(Hd), 4, 0, 128, scales_in=s)
    assert np.array_equal(g["codes"], r["codes"])


# ---------------------------------------------------------------------------------- f3: AWQ scaling
def test_awq_search_pins():
    rng = np.random.default_rng(95)
    n, m, N = 64, 40, 500
    X = rng.standard_normal((N, n))
    X[:, 5] *= 30.0                                          # one salient input channel
    X[:, 9] = 0.0                                            # a dead channel: s = 1
    W = rng.normal(0, 0.02, size=(m, n))
    # channel means by brute force
    a = O.channel_abs_mean([X[:200], X[200:]])
    for c in (0, 5, 9):
        assert abs(a[c] - sum(abs(X[t, c]) for t in range(N)) / N) <= 1e-12 * max(1.0, a[c])
    res = O.awq_search(W, X, 4, 16, n_alpha=11)
    # alpha = 0 is plain RTN, exactly
    r0 = O.rtn(W, 4, 16)
    assert res["mse"][0] == O.recon_mse(X, W, r0["What"])
    assert res["mse"][res["best"]] <= res["mse"][0]
    # every candidate's score is the trace identity with H
    H = O.hessian(X)
    for k in (0, 4, 10):
        s = O.awq_scales(a, k / 10)
        rk = O.rtn(W * s, 4, 16)
        dW_what = rk["What"] / s
        assert abs(res["mse"][k] - O.recon_mse_trace(H, N, W, dW_what)) <= 1e-9 * res["mse"][k]
    # the transformation leaves the layer unchanged before quantization: (X / s) (W s)^T = X W^T
    s = res["s"]
    assert np.allclose((X / s) @ (W * s).T, X @ W.T, rtol=1e-12, atol=1e-12)
    assert s[9] == 1.0
    # the salient channel is protected: its weights' error shrinks against plain RTN
    e_awq = np.abs(W[:, 5] - res["What"][:, 5]).mean()
    e_rtn = np.abs(W[:, 5] - r0["What"][:, 5]).mean()
    assert res["best"] > 0 and e_awq < e_rtn


def test_forced_replay_of_own_codes_is_silent_and_flags_a_planted_flip():
    """Replaying the oracle's own decisions changes nothing; a planted code flip is reported
    with its distance from the rounding boundary."""
    rng = np.random.default_rng(98)
    m, n = 40, 96
    X = ar1_x(rng, 300, n, 0.8)
    W = rng.normal(0, 0.02, size=(m, n))
    Hd, _ = O.damp_hessian(O.hessian(X), 0.01)
    U = O.chol_inverse_upper(Hd)
    for sym in (True, False):
        ref = O.gptq(W, U, 4, 32, 32, sym=sym)
        rep = O.gptq(W, U, 4, 32, 32, sym=sym, forced_codes=ref["codes"], forced_scales=ref["scales"],
                     forced_zeros=ref["zeros"])
        assert rep["forced"]["count"] == 0 and np.array_equal(rep["codes"], ref["codes"])
        assert rep["forced"]["scale_mismatch"] == 0 and rep["forced"]["groups"] == m * 3
        bad = ref["codes"].astype(np.int64).copy()
        hi = 7 if sym else 15
        bad[3, 40] = bad[3, 40] - 1 if bad[3, 40] > (-7 if sym else 0) else bad[3, 40] + 1
        rep2 = O.gptq(W, U, 4, 32, 32, sym=sym, forced_codes=bad)
        assert rep2["forced"]["count"] >= 1 and rep2["forced"]["max_step"] == 1
        assert 0.0 <= rep2["forced"]["max_distance"] <= 1.0 + 1e-9
        assert rep2["codes"][3, 40] == bad[3, 40] and abs(int(bad[3, 40])) <= hi
