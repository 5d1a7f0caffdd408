"""The pins catch plausible mistakes: each test plants one in the oracle's inputs or code
path (on the CPU) and checks that a pin fails for it."""
import numpy as np
import pytest

import oracle as O
from test_oracle_pins import ar1_x, tril_ones
from conftest import read_golden


def _setup(seed=21, n=8, rows=300, bits=3):
    rng = np.random.default_rng(seed)
    X = ar1_x(rng, 64, n)
    W = rng.normal(0, 0.02, size=(rows, n))
    Hd, _ = O.damp_hessian(O.hessian(X), 0.01)
    U = O.chol_inverse_upper(Hd)
    ref = O.direct_obs(W, Hd, bits, 0)
    return W, Hd, U, ref, bits


def _agree(a, b):
    return float(np.mean(a == b))


def test_full_inverse_reading_fails_direct_obs_pin():
    """Using rows of the full H^-1 (the listing's literal form) instead of its Cholesky factor."""
    W, Hd, U, ref, bits = _setup()
    Hinv = np.linalg.inv(Hd)
    wrong = O.gptq(W, np.triu(Hinv), bits, 0, 128)
    assert _agree(wrong["codes"], ref["codes"]) < 0.99
    assert np.array_equal(O.gptq(W, U, bits, 0, 128)["codes"], ref["codes"])


def test_transposed_factor_fails():
    W, Hd, U, ref, bits = _setup()
    wrong = O.gptq(W, U.T.copy(), bits, 0, 128)      # lower triangle: the loop sees no updates
    assert _agree(wrong["codes"], ref["codes"]) < 0.99


def test_sign_flip_fails():
    W, Hd, U, ref, bits = _setup()
    Uf = -U
    Uf[np.diag_indices_from(Uf)] *= -1               # off-diagonal sign flipped
    wrong = O.gptq(W, Uf, bits, 0, 128)
    assert _agree(wrong["codes"], ref["codes"]) < 0.99


def test_dropped_diagonal_scaling_fails():
    W, Hd, U, ref, bits = _setup()
    Ud = U.copy()
    Ud[np.diag_indices_from(Ud)] = 1.0               # e = (w - what) without / U_jj
    wrong = O.gptq(W, Ud, bits, 0, 128)
    assert _agree(wrong["codes"], ref["codes"]) < 0.99


def test_off_by_one_row_fails_carry_example():
    """Reading row j+1 of U for column j's update breaks the lesson's worked example."""
    g = read_golden("lesson17_example_1_1.txt")
    w = np.array([g["weights"]])
    Hd, _ = O.damp_hessian(O.hessian(tril_ones(6)), 0.0)
    U = O.chol_inverse_upper(Hd)
    Ushift = np.zeros_like(U)
    Ushift[:-1, 1:] = U[1:, 1:]
    Ushift[np.diag_indices_from(Ushift)] = np.diag(U)
    s = np.array([[g["step"]]], dtype=np.float16)
    out = O.gptq(w, np.triu(Ushift), 4, 0, 128, scales_in=s)["What"][0]
    assert [round(v, 1) for v in out] != g["compensated"]


def test_missing_factor_two_in_hessian_is_harmless_but_damping_matters():
    """Codes do not depend on a positive factor on H (relative damping); an absolute damping
    constant instead of damp * mean(diag H) changes them."""
    rng = np.random.default_rng(22)
    n, m = 32, 64
    X = ar1_x(rng, 128, n, 0.9)
    W = rng.normal(0, 0.02, size=(m, n))
    H = O.hessian(X)
    Hd, lam = O.damp_hessian(H, 0.01)
    a = O.gptq(W, O.chol_inverse_upper(Hd), 4, 0, 8)
    Hh, _ = O.damp_hessian(H / 2, 0.01)
    b = O.gptq(W, O.chol_inverse_upper(Hh), 4, 0, 8)
    assert np.array_equal(a["codes"], b["codes"])
    Habs = H + 50.0 * lam * np.eye(n)
    c = O.gptq(W, O.chol_inverse_upper(Habs), 4, 0, 8)
    assert not np.array_equal(a["codes"], c["codes"])


@pytest.mark.parametrize("bad", ["scale_no_fp16", "ceil_scale"])
def test_scale_rule_mistakes_change_codes(bad):
    rng = np.random.default_rng(23)
    W = rng.normal(0, 0.02, size=(256, 256)).astype(np.float32)
    good = O.rtn(W, 4, 128)
    a = np.stack([np.max(np.abs(W[:, :128]), 1), np.max(np.abs(W[:, 128:]), 1)], 1).astype(np.float64)
    if bad == "scale_no_fp16":
        # keep the float32 quotient: stored scale and codes change against the 16-bit format
        s = (a.astype(np.float32) / np.float32(7)).astype(np.float64)
        assert not np.array_equal(s, good["scales"].astype(np.float64))
    else:
        s = a / 7.5                                   # 16 levels instead of 15
        wrong = O.rtn(W, 4, 128, scales_in=s.astype(np.float16))
        assert not np.array_equal(wrong["codes"], good["codes"])
