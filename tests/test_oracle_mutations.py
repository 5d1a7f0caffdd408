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


# ---------------------------------------------------------------------------------- zero-points
import oracle.pwq_oracle as OM
import test_oracle_pins as P


def _wrong_zero_sign(lo, hi, bits):
    s, z = _good_scale_zero(lo, hi, bits)
    top = (1 << bits) - 1
    lo32 = np.asarray(lo, dtype=np.float64).astype(np.float32).astype(np.float64)
    safe = np.where(s.astype(np.float64) > 0, s.astype(np.float64), 1.0)
    return s, np.clip(np.rint(lo32 / safe), 0, top).astype(np.uint16)


def _wrong_zero_floor(lo, hi, bits):
    s, _ = _good_scale_zero(lo, hi, bits)
    lo32 = np.asarray(lo, dtype=np.float64).astype(np.float32).astype(np.float64)
    safe = np.where(s.astype(np.float64) > 0, s.astype(np.float64), 1.0)
    z = np.where(s.astype(np.float64) > 0, np.floor(-lo32 / safe), 0)
    return s, np.clip(z, 0, (1 << bits) - 1).astype(np.uint16)


def _wrong_levels(lo, hi, bits):
    """2^b levels spaced by range / 2^b (one level too many)."""
    span = (np.asarray(hi, np.float64) - np.asarray(lo, np.float64)).astype(np.float32)
    s = (span / np.float32(1 << bits)).astype(np.float16)
    sf = s.astype(np.float64)
    z = np.where(sf > 0, np.rint(-np.asarray(lo, np.float64) / np.where(sf > 0, sf, 1)), 0)
    return s, np.clip(z, 0, (1 << bits) - 1).astype(np.uint16)


def _wrong_codes_no_zero(w, s16, z, bits):
    return _good_codes(w, s16, np.zeros_like(np.asarray(z)), bits)


_good_scale_zero = OM.asym_scale_zero
_good_codes = OM.quantize_codes_asym


@pytest.mark.parametrize("target,bad", [
    ("asym_scale_zero", _wrong_zero_sign),
    ("asym_scale_zero", _wrong_zero_floor),
    ("asym_scale_zero", _wrong_levels),
    ("quantize_codes_asym", _wrong_codes_no_zero),
])
def test_zero_point_mistakes_fail_a_pin(monkeypatch, target, bad):
    monkeypatch.setattr(OM, target, bad)
    failed = 0
    for pin in (P.test_asym_worked_group, P.test_asym_scale_zero_closed_form):
        try:
            if pin is P.test_asym_scale_zero_closed_form and target != "asym_scale_zero":
                continue
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_dequant_without_zero_fails_nearest_level_pin(monkeypatch):
    def bad_dequant(codes, scales, group_size, g_idx=None, out_dtype=np.float64, zeros=None):
        return _good_dequant(codes, scales, group_size, g_idx=g_idx, out_dtype=out_dtype, zeros=None)
    _good_dequant = OM.dequant
    monkeypatch.setattr(OM, "dequant", bad_dequant)
    with pytest.raises(AssertionError):
        P.test_asym_worked_group()


def test_offset_nibble_fails_unsigned_pack_pin(monkeypatch):
    """Zero-point codes packed with the symmetric layout's +8 offset."""
    def bad_pack(c):
        u = ((np.asarray(c, np.int16) + 8) & 15).astype(np.uint8)
        return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    monkeypatch.setattr(O, "pack_uint4", bad_pack)
    with pytest.raises(AssertionError):
        P.test_asym_pack_layout_and_storage()


def test_awq_wrong_scale_direction_fails_pin(monkeypatch):
    """Shrinking the salient channel (s = a^-alpha) instead of growing it."""
    good = OM.awq_scales
    monkeypatch.setattr(OM, "awq_scales", lambda a, alpha: good(a, -alpha))
    with pytest.raises(AssertionError):
        P.test_awq_search_pins()


def test_awq_unscaled_reconstruction_fails_pin(monkeypatch):
    """Scoring W diag(s)'s quantization without dividing by s again."""
    def bad_search(W, x_tiles, bits=4, group_size=128, n_alpha=21, sym=True):
        res = good(W, x_tiles, bits, group_size, n_alpha, sym)
        X = x_tiles if isinstance(x_tiles, np.ndarray) else np.concatenate(list(x_tiles))
        a = OM.channel_abs_mean(X)
        for k in range(n_alpha):
            s = OM.awq_scales(a, k / (n_alpha - 1))
            res["mse"][k] = OM.recon_mse(X, W, OM.rtn(np.asarray(W) * s, bits, group_size, sym=sym)["What"])
        return res
    good = OM.awq_search
    monkeypatch.setattr(O, "awq_search", bad_search)
    with pytest.raises(AssertionError):
        P.test_awq_search_pins()


# ---------------------------------------------------------------------------------- whole layer
import test_oracle_layer_pins as LP


def _layer_with(mistake):
    """quantize_layer's composition with one planted mistake."""
    def layer(W, x_tiles, bits=4, group_size=128, block_size=128, damp=0.01, act_order=False, perm=None,
              sym=True):
        if isinstance(x_tiles, np.ndarray):
            x_tiles = [x_tiles]
        x_tiles = list(x_tiles)
        H = OM.hessian(x_tiles)
        n_tok = sum(int(np.asarray(t).shape[0]) for t in x_tiles)
        Hd, lam = OM.damp_hessian(H, damp)
        if mistake == "undamped_factor":
            Hd = H + 1e-300 * np.eye(H.shape[0])
        if act_order and perm is None:
            perm = OM.act_order_perm(Hd)
        elif not act_order:
            perm = None
        Hp = Hd[np.ix_(perm, perm)] if (perm is not None and mistake != "perm_on_w_only") else Hd
        U = OM.chol_inverse_upper(Hp)
        res = OM.gptq(W, U, bits, group_size, block_size, perm=perm, sym=sym)
        r = OM.rtn(W, bits, group_size, sym=sym)
        What = res["What"]
        if mistake == "what_in_processing_order" and perm is not None:
            What = What[:, perm]
        res.update({"H": H, "lambda": lam, "perm": perm, "U": U, "rtn": r, "n_tok": n_tok,
                    "gptq_mse": OM.recon_mse(x_tiles, W, What), "rtn_mse": OM.recon_mse(x_tiles, W, r["What"])})
        return res
    return layer


LAYER_PINS = [LP.test_layer_diagonal_hessian_is_rtn, LP.test_layer_sorted_diagonal_act_order_is_identity,
              LP.test_layer_errors_brute_force, LP.test_layer_two_column_compensation_closed_form,
              LP.test_layer_damping_makes_rank_deficient_inputs_factorable]
PIN_ARGS = {LP.test_layer_diagonal_hessian_is_rtn: [(0,), (32,)], LP.test_layer_errors_brute_force: [(False,), (True,)],
            LP.test_layer_two_column_compensation_closed_form: [(1,), (128,)]}


def _failing_layer_pins():
    failed = []
    for pin in LAYER_PINS:
        for args in PIN_ARGS.get(pin, [()]):
            try:
                pin(*args)
            except (AssertionError, ArithmeticError, np.linalg.LinAlgError):
                failed.append(pin.__name__)
    return failed


def test_unmutated_layer_passes_every_layer_pin(monkeypatch):
    monkeypatch.setattr(O, "quantize_layer", _layer_with(None))
    assert _failing_layer_pins() == []


@pytest.mark.parametrize("mistake", ["perm_on_w_only", "undamped_factor", "what_in_processing_order"])
def test_layer_composition_mistakes_fail_a_pin(monkeypatch, mistake):
    monkeypatch.setattr(O, "quantize_layer", _layer_with(mistake))
    assert _failing_layer_pins(), mistake
