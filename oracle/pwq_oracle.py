"""Plain float64 CPU oracle for layer-wise post-training weight quantization.

TEST INFRASTRUCTURE.  This module is the checker the GPU library is compared
against.  It is deliberately slow and literal: numpy in float64, one step of the
method per function, no blocking, fusion or reordering beyond what the method
itself states.  It shares no code with the HIP library.

Sources (page title, then section):

* [GPT2-RE]  "GPT-2 Quantization Reconstruction Error", sections "What this
  project does" and "Setup": 4-bit symmetric quantization with one scale per
  output row (channel), rounded to 15 levels and dequantized; per-layer output MSE.
* [MQM]      "Model Quantization Mechanics: Precision Reduction and Weight
  Formatting", section 1 ("Affine Quantization", "Group-wise Quantization") and
  section 2.1 (GPTQ objective, Cholesky factor of the inverse Hessian).
* [LESSON17] "17 - GPTQ and AWQ" (Inference and Serving), Part 1, "Your turn" and
  Example 1.1 "Rounding with the error carried forward".
* [GPTQ-P]   "GPTQ: Post-Training INT4", sections "OBQ Foundation",
  "Hessian-Based Weight Update", "The GPTQ Algorithm", "Group Quantization",
  "Running GPTQ with AutoGPTQ" (config knobs group_size, desc_act, damp_percent, sym).
* [SWEEP]    "Quantization sweep: perplexity vs compression", "How I ran each
  one" (damp_percent 0.0 for RTN, 0.01 for GPTQ, group size 128).

Readings taken where the pages are silent, ambiguous or garbled (each is also
listed in the design notes):

* R1  The factor that drives the column loop is U, the upper-triangular Cholesky
      factor of H^-1 (H^-1 = U^T U), as [MQM] 2.1 states.  The code listing in
      [GPTQ-P] indexes the full H^-1 instead; that literal form is exact only for the
      first column and is not taken.  Only the U form makes each step the OBS
      update on the still-unquantized set (``direct_obs`` checks this).
* R2  The OBS update printed in [GPTQ-P] "Hessian-Based Weight Update" uses entries
      of H where the optimum needs the inverse restricted to the free set; we follow
      the listing's signs: e = (w - what) / U_jj, then w_k -= e * U_jk for k > j.
* R3  Damping: lambda = damp * mean(diag H) of the undamped H, added to every
      diagonal entry ([GPTQ-P] "Running GPTQ with AutoGPTQ", damp_percent; damp may
      be 0 as in [SWEEP]).
* R4  H = 2 X^T X with X stored tokens x d_in, summed (not averaged) over tokens
      ([GPTQ-P] "Hessian-Based Weight Update" and the listing; codes do not depend
      on a positive factor on H when the damping is relative).
* R5  A group's scale is taken, when the loop reaches the group's first column,
      from the current (error-updated) values of the group's columns.  With one
      scale per row that is the original row.
* R6  The listing's "q" in (w - q) / h_inv_jj is the dequantized value s * code.
* R7  Scale: s = fp16( fp32( fp32(absmax) / qmax ) ), qmax = 2^(bits-1) - 1, i.e. one
      IEEE float32 division rounded to float16 (the stored 16-bit scale of
      [GPTQ-P] "Group Quantization"); codes are computed against the stored scale.
* R8  Codes: nearest integer to the exact quotient w / s, ties to even (Python's
      round, as in [LESSON17]'s listing), clamped to [-qmax, qmax] (15 levels for
      4 bits, [GPT2-RE]); an all-zero group has s = 0 and all codes 0.
* R9  Act-order (desc_act): columns processed by descending diag H (stable: lower
      original index first on ties); groups are consecutive in processing order;
      codes are returned in original column order with g_idx[c] = position(c) // g.
* R10 INT4 storage: nibble u = code + 8; byte k of a row holds column 2k in the low
      nibble and column 2k+1 in the high nibble.
* R11 Reconstruction MSE: mean over all tokens x outputs of (X (W - What)^T)^2 with the
      same X for both and the original W ([GPT2-RE] step 5, per layer).
* R12 A non positive definite H raises NotPositiveDefinite (no automatic re-damping).
* A1  Zero-point (asymmetric) quantization, [MQM] "Affine Quantization": code =
      round(w / S) + Z, dequantized S (code - Z).  The pages give no rule for S and Z;
      the plainest one that keeps real 0 exact: a group's range [lo, hi] = [min(w, 0),
      max(w, 0)] is mapped onto the codes 0 .. 2^b - 1.
* A2  S = fp16( fp32( fp32(hi - lo) / (2^b - 1) ) ) (one float32 subtraction and one
      float32 division, then float16, as R7).
* A3  Z = round(-lo / S) (exact quotient, ties to even), clamped to [0, 2^b - 1]; stored in
      16 bits as [GPTQ-P] "Group Quantization" counts it (4 + 32/g bits per weight).  S = 0
      (an all-zero group, or a range below float16) gives Z = 0 and every code 0.
* A4  Codes: clamp(round(w / S) + Z, 0, 2^b - 1), round = nearest integer to the exact
      quotient, ties to even (R8); INT4 nibble = code itself (R10's layout otherwise).
* A5  GPTQ with zero-points takes S and Z at a group's first column from the current
      values of the group's columns (R5), and the dequantized value S (code - Z) (R6).
* T1  Per-tensor quantization ([GPT2-RE] "Possible extensions": per-channel against a single
      global scale): one quantizer for the whole matrix, taken from the original W like the
      per-row one (R5), by the per-row rules (R7, A2-A3) applied to the whole tensor; it is
      stored as the per-row format with every row holding the same scale (and zero).
* W1  Activation-aware channel scaling ([MQM] 2.2 "AWQ": salience from the size of a column's
      input activations; W's column multiplied and X's column divided by a per-channel s, the
      layer output unchanged; [GPT2-RE] "Possible extensions": scale up the important
      channels before quantizing).  The pages give no rule for s.  Reading taken: the size
      of input channel c is a_c = mean over tokens of |X_tc| (a_c = 0 gives s_c = 1),
      s_c = a_c^alpha, alpha on the grid k / (K - 1), k = 0 .. K - 1 (alpha = 0 is plain
      RTN); for each alpha, RTN of W diag(s), What = dequant / s column-wise, scored by the
      reconstruction MSE with the original W and X (R11); the least MSE wins, ties to the
      smaller alpha.
* G1  The product with the quantized weights ([GPTQ-P] "Running GPTQ with AutoGPTQ": the
      quantized model runs inference on them) is Y = X What^T, What decoded exactly as in
      ``dequant``; tokens x d_in times d_out x d_in gives tokens x d_out.

Pins (tests/test_oracle_pins.py):
  rtn / quantize_codes / group_scales : golden tie-to-even rows, code range, error bound,
                                        level count
  gptq / gptq_unblocked               : [LESSON17] worked examples (golden) and the carry
                                        rule's closed form, diagonal-H == rtn, direct_obs
                                        agreement, batched == unblocked for every block
                                        size, scale invariance, brute-force optimum on tiny rows
  chol_inverse_upper                  : U^T U H = I, triangular, positive diagonal,
                                        reverse-order Cholesky + triangular inverse route
  hessian / damp                      : brute force on tiny X, trace identity, symmetry
  act_order_perm                      : already-sorted diagonal == no act-order; g_idx round trip
  pack_int4 / dequant                 : golden bytes, storage bits/weight of [GPTQ-P]
  recon_mse                           : trace identity with the undamped Hessian
  asym_scale_zero / rtn_asym / gptq(sym=False) : golden worked group (A1-A4), exact zero,
                                        error bound, range end points, 4.25 bits/weight,
                                        diagonal-H == rtn_asym, block-size invariance
  quantized_matmul                    : brute-force sums on tiny inputs, identity X gives
                                        What^T, rows of X against hand-dequantized rows
  channel_abs_mean / awq_search       : brute-force column means; alpha = 0 reproduces RTN
                                        exactly; every candidate's score equals the trace
                                        identity with H; the output of X / s through W s is
                                        X W^T; an outlier channel is protected
  quantize_layer                      : (tests/test_oracle_layer_pins.py) the OBS compensation
                                        on a two-column block in exact rationals, with and
                                        without act-order; diagonal H == RTN (of the permuted
                                        matrix with act-order); a sorted diagonal leaves
                                        act-order a no-op; both errors by brute-force sums;
                                        rank-deficient X factorable only with damping
  tensor_scales                       : the per-row rule on the flattened matrix; the
                                        tensor's absmax element maps to +-qmax; GPTQ with a
                                        diagonal H and these scales equals RTN with them
"""
from __future__ import annotations

from typing import Iterable, Optional, Union

import numpy as np

__all__ = [
    "NotPositiveDefinite", "qmax", "group_scales_from_absmax", "quantize_codes",
    "hessian", "damp_hessian", "act_order_perm", "chol_inverse_upper",
    "gptq", "gptq_unblocked", "rtn", "pack_int4", "unpack_int4", "dequant",
    "recon_mse", "recon_mse_trace", "direct_obs", "quantize_layer", "n_groups",
    "storage_bytes", "asym_scale_zero", "quantize_codes_asym", "rtn_asym", "dequant_asym",
    "pack_uint4", "unpack_uint4", "quantized_matmul", "tensor_scales", "channel_abs_mean",
    "awq_scales", "awq_search",
]


class NotPositiveDefinite(ArithmeticError):
    """H (after damping) is not positive definite; ``pivot`` is the 0-based failing pivot
    in reverse column order (the order the GPU factorization eliminates in)."""

    def __init__(self, pivot: int):
        super().__init__(f"Hessian not positive definite (pivot {pivot})")
        self.pivot = pivot


# ------------------------------------------------------------------ quantizer primitives

def qmax(bits: int) -> int:
    """Largest code magnitude: 7 for 4 bits, i.e. 15 levels -7..7 ([GPT2-RE], R8)."""
    return (1 << (bits - 1)) - 1


def n_groups(d_in: int, group_size: int) -> int:
    return 1 if group_size == 0 else -(-d_in // group_size)


def group_scales_from_absmax(absmax: np.ndarray, bits: int) -> np.ndarray:
    """Symmetric scale S of [MQM] "Affine Quantization" with Z = 0: absmax / qmax,
    as one float32 division, stored as float16 (R7).  Returns float16."""
    a32 = np.asarray(absmax, dtype=np.float64).astype(np.float32)
    s32 = (a32 / np.float32(qmax(bits))).astype(np.float32)
    return s32.astype(np.float16)


def quantize_codes(w: np.ndarray, s16: np.ndarray, bits: int) -> np.ndarray:
    """Codes round(w / s) ([MQM] "Affine Quantization", Z = 0), exact quotient rounded to
    nearest-even in float64, clamped to +-qmax; s = 0 gives code 0 (R8).

    float64 decides these exactly: w has at most 24 significant bits and s 11, so a
    quotient that is not a tie lies at least 2^-29 (relative) from k + 1/2, far above
    float64's division error."""
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    safe = np.where(s > 0, s, 1.0)
    q = np.rint(w / safe)
    q = np.clip(q, -qmax(bits), qmax(bits))
    q = np.where(s > 0, q, 0.0)
    return q.astype(np.int8)


def asym_scale_zero(lo: np.ndarray, hi: np.ndarray, bits: int):
    """Scale and zero-point of [MQM] "Affine Quantization" for a range [lo, hi] that holds 0
    (A1-A3): S = fp16(fp32(fp32(hi - lo) / (2^b - 1))), Z = round(-lo / S) clamped to
    [0, 2^b - 1], Z = 0 where S = 0.  Returns (S float16, Z uint16)."""
    top = (1 << bits) - 1
    lo32 = np.asarray(lo, dtype=np.float64).astype(np.float32)
    hi32 = np.asarray(hi, dtype=np.float64).astype(np.float32)
    span = (hi32 - lo32).astype(np.float32)
    s16 = (span / np.float32(top)).astype(np.float32).astype(np.float16)
    s = s16.astype(np.float64)
    safe = np.where(s > 0, s, 1.0)
    z = np.clip(np.rint(-lo32.astype(np.float64) / safe), 0, top)
    z = np.where(s > 0, z, 0.0)
    return s16, z.astype(np.uint16)


def quantize_codes_asym(w: np.ndarray, s16: np.ndarray, z: np.ndarray, bits: int) -> np.ndarray:
    """Codes round(w / S) + Z clamped to [0, 2^b - 1] (A4); the quotient is decided exactly
    as in ``quantize_codes``.  S = 0 gives code 0.  Returns uint8."""
    top = (1 << bits) - 1
    w = np.asarray(w, dtype=np.float64)
    s = np.asarray(s16, dtype=np.float16).astype(np.float64)
    zz = np.asarray(z, dtype=np.float64)
    safe = np.where(s > 0, s, 1.0)
    q = np.clip(np.rint(w / safe) + zz, 0, top)
    q = np.where(s > 0, q, 0.0)
    return q.astype(np.uint8)


def _pre_scale(vals: np.ndarray, bits: int, sym: bool) -> np.ndarray:
    """The float32 quotient a group's stored scale rounds to float16 (R7, A2), float64."""
    if sym:
        a32 = np.max(np.abs(vals), axis=1).astype(np.float32)
        return (a32 / np.float32(qmax(bits))).astype(np.float32).astype(np.float64)
    lo32 = np.minimum(np.min(vals, axis=1), 0.0).astype(np.float32)
    hi32 = np.maximum(np.max(vals, axis=1), 0.0).astype(np.float32)
    span = (hi32 - lo32).astype(np.float32)
    return (span / np.float32((1 << bits) - 1)).astype(np.float32).astype(np.float64)


def _group_params(vals: np.ndarray, bits: int, sym: bool):
    """Per-row quantizer of a group from its current values (rows x columns): the
    symmetric scale (R7), or the zero-point pair of A1-A3."""
    if sym:
        return group_scales_from_absmax(np.max(np.abs(vals), axis=1), bits), None
    lo = np.minimum(np.min(vals, axis=1), 0.0)
    hi = np.maximum(np.max(vals, axis=1), 0.0)
    return asym_scale_zero(lo, hi, bits)


def tensor_scales(W: np.ndarray, bits: int, sym: bool = True):
    """One quantizer for the whole matrix (T1), replicated per row: (scales d_out x 1
    float16, zeros d_out x 1 uint16 or None).  Use with group_size 0 and fixed scales."""
    W = np.asarray(W, dtype=np.float64)
    m = W.shape[0]
    flat = W.reshape(1, -1)
    s, z = _group_params(flat, bits, sym)
    scales = np.full((m, 1), s[0], dtype=np.float16)
    zeros = None if sym else np.full((m, 1), z[0], dtype=np.uint16)
    return scales, zeros


def _codes(w, s16, z, bits: int, sym: bool):
    return quantize_codes(w, s16, bits) if sym else quantize_codes_asym(w, s16, z, bits)


def _value(s16, z, q) -> np.ndarray:
    """The dequantized value S (q - Z) in float64 (exact)."""
    v = np.asarray(q, dtype=np.float64)
    if z is not None:
        v = v - np.asarray(z, dtype=np.float64)
    return np.asarray(s16, dtype=np.float16).astype(np.float64) * v


# ------------------------------------------------------------------ Hessian, damping, order

def hessian(x_tiles: Union[np.ndarray, Iterable[np.ndarray]]) -> np.ndarray:
    """H = 2 X^T X, summed over all tokens ([GPTQ-P] "Hessian-Based Weight Update", R4).

    ``x_tiles`` is X (tokens x d_in) or an iterable of token tiles; values are taken
    in float64 exactly as stored."""
    if isinstance(x_tiles, np.ndarray):
        x_tiles = [x_tiles]
    H = None
    for xt in x_tiles:
        x = np.asarray(xt, dtype=np.float64)
        part = x.T @ x
        H = part if H is None else H + part
    return 2.0 * H


def damp_hessian(H: np.ndarray, damp: float):
    """H + lambda I with lambda = damp * mean(diag H) (R3).  Returns (H_damped, lambda)."""
    lam = float(damp) * float(np.mean(np.diag(H)))
    Hd = H.copy()
    Hd[np.diag_indices_from(Hd)] += lam
    return Hd, lam


def act_order_perm(H: np.ndarray) -> np.ndarray:
    """Processing order for desc_act: descending diag H, stable on ties (R9)."""
    return np.argsort(-np.diag(H), kind="stable").astype(np.int32)


def chol_inverse_upper(H: np.ndarray) -> np.ndarray:
    """U upper triangular with H^-1 = U^T U and U_jj > 0 ([MQM] 2.1, R1).

    Textbook route: the Cholesky factor of H (H = R^T R), H^-1 from it (LAPACK potri),
    then the lower Cholesky factor L of H^-1, U = L^T.  Raises NotPositiveDefinite when H
    is not positive definite (R12); the pivot is then located by LAPACK's Cholesky of H in
    reversed index order, the order the GPU factorization eliminates in."""
    from scipy.linalg import lapack

    n = H.shape[0]
    R, info = lapack.dpotrf(np.array(H, dtype=np.float64, order="F"), lower=0, clean=1, overwrite_a=1)
    if info != 0:
        rev = H[::-1, ::-1]
        _, info_r = lapack.dpotrf(np.array(rev, dtype=np.float64, order="F"), lower=1)
        k = int(info_r) - 1 if info_r > 0 else max(int(info) - 1, 0)
        raise NotPositiveDefinite(n - 1 - k)
    S, info = lapack.dpotri(R, lower=0, overwrite_c=1)      # upper triangle of H^-1
    if info != 0:
        raise NotPositiveDefinite(n - 1)
    del R
    S = np.triu(S)
    S += np.triu(S, 1).T                                     # H^-1, both triangles
    L, info = lapack.dpotrf(S, lower=1, clean=1, overwrite_a=1)
    if info != 0:
        raise NotPositiveDefinite(n - 1)
    return np.ascontiguousarray(L.T)


# ------------------------------------------------------------------ GPTQ column loop

def _group_len(n: int, group_size: int) -> int:
    return n if group_size == 0 else group_size


def _finish(codes_p, scales, perm, group_size, bits, zeros=None):
    m, n = codes_p.shape
    if perm is None:
        codes, g_idx = codes_p, None
    else:
        codes = np.empty_like(codes_p)
        codes[:, perm] = codes_p
        g = _group_len(n, group_size)
        g_idx = np.empty(n, dtype=np.int32)
        g_idx[perm] = (np.arange(n) // g).astype(np.int32)
    What = dequant(codes, scales, group_size, g_idx=g_idx, out_dtype=np.float64, zeros=zeros)
    return {"codes": codes, "scales": scales, "zeros": zeros, "g_idx": g_idx, "What": What,
            "bits": bits, "group_size": group_size}


def _init_params(m, ng, scales_in, zeros_in, sym):
    scales = np.zeros((m, ng), dtype=np.float16) if scales_in is None else np.array(scales_in, dtype=np.float16).reshape(m, ng)
    if sym:
        return scales, None
    if scales_in is not None and zeros_in is None:
        raise ValueError("zero-point quantization with given scales needs the zeros too")
    zeros = np.zeros((m, ng), dtype=np.uint16) if zeros_in is None else np.array(zeros_in, dtype=np.uint16).reshape(m, ng)
    return scales, zeros


def _current(Wp: np.ndarray, E: np.ndarray, U: np.ndarray, j: int, c0: int, c1: int) -> np.ndarray:
    """Values of columns c0..c1-1 once columns 0..j-1 are fixed: each fixed column i has
    moved every later column k by -e_i U_ik (R1, R2), so the current value is the original
    one less sum_i e_i U_ik over the fixed columns."""
    if j == 0:
        return Wp[:, c0:c1].copy()
    return Wp[:, c0:c1] - E[:, :j] @ U[:j, c0:c1]


def gptq(W: np.ndarray, U: np.ndarray, bits: int = 4, group_size: int = 128, block_size: int = 128,
         perm: Optional[np.ndarray] = None, scales_in: Optional[np.ndarray] = None,
         sym: bool = True, zeros_in: Optional[np.ndarray] = None,
         forced_codes: Optional[np.ndarray] = None, forced_scales: Optional[np.ndarray] = None,
         forced_zeros: Optional[np.ndarray] = None) -> dict:
    """GPTQ in fixed left-to-right order with the updates applied in batches ([GPTQ-P] "The
    GPTQ Algorithm", R1-R9).

    W: d_out x d_in (any float dtype, promoted to float64).  U: the factor of
    ``chol_inverse_upper`` of the (damped, permuted if ``perm``) Hessian.

    Column j is quantized at its current value: the original value less e_i U_ij for every
    column i < j already fixed, where e_i = (w_i - what_i) / U_ii is column i's error scaled
    by the factor's diagonal.  This is ``gptq_unblocked`` (every error pushed to all later
    columns at once) with the sums regrouped, which the pages' lazy batching amounts to:
    the errors of all earlier blocks of ``block_size`` columns reach a block in one product
    when the block starts; inside the block each column adds the terms of the block's
    earlier columns.  A group's scale (and zero) is taken at its first column from the
    current values of all its columns, including any past the block (R5).

    ``sym=False``: zero-point quantization (A1-A5); the group's scale and zero come from
    the same current values the symmetric scale would.

    ``forced_codes`` (d_out x d_in, processing order): a replay of another run's decisions.
    Every column is quantized as above, but the code taken - and so the error carried on -
    is the given one; where it differs from this function's own, ``forced`` records the
    distance of the exact quotient (plus the zero) from the rounding boundary between the
    two codes, in units of the scale (0 at an exact tie).  ``forced_scales`` (and
    ``forced_zeros``) likewise replace each group's quantizer once this function has taken
    its own and recorded how far apart the two are (float16 ulps, and for a differing scale
    the relative distance of its float32 quotient from the float16 rounding boundary between
    the two).  The arithmetic is otherwise unchanged;
    it checks that the other run decided like this one given the same history.

    Rows are independent (each row has its own scales and sees the same U), so a subset of
    rows gives the same result for those rows as the whole matrix.

    Returns codes (int8, or uint8 with zero-points; original column order), scales
    (float16, d_out x groups, in processing order), zeros (uint16 like scales, or None),
    g_idx (int32 or None) and What (float64)."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    Wp = W[:, perm].copy() if perm is not None else W.copy()
    g = _group_len(n, group_size)
    ng = n_groups(n, group_size)
    scales, zeros = _init_params(m, ng, scales_in, zeros_in, sym)
    codes_p = np.zeros((m, n), dtype=np.int8 if sym else np.uint8)
    E = np.zeros((m, n))
    B = int(block_size)
    forced = None
    if forced_codes is not None:
        forced = {"count": 0, "max_distance": 0.0, "max_step": 0, "groups": 0, "scale_mismatch": 0,
                  "scale_max_ulp": 0, "scale_max_distance": 0.0, "zero_mismatch": 0, "zero_max_step": 0}
    for b0 in range(0, n, B):
        b1 = min(b0 + B, n)
        cur = _current(Wp, E, U, b0, b0, b1)            # every earlier block's errors, one product
        for j in range(b0, b1):
            G = j // g
            if j % g == 0 and scales_in is None:
                vals = _current(Wp, E, U, j, j, min(j + g, n))
                sG, zG = _group_params(vals, bits, sym)
                if forced is not None and forced_scales is not None:
                    fs = np.asarray(forced_scales, dtype=np.float16).reshape(m, ng)[:, G]
                    d = np.abs(fs.view(np.uint16).astype(np.int64) - sG.view(np.uint16).astype(np.int64))
                    forced["groups"] += m
                    forced["scale_mismatch"] += int((d != 0).sum())
                    forced["scale_max_ulp"] = max(forced["scale_max_ulp"], int(d.max()))
                    if (d != 0).any():
                        # relative distance of this function's float32 quotient from the float16
                        # rounding boundary between the two scales (their midpoint when they are
                        # neighbours)
                        pre = _pre_scale(vals[d != 0], bits, sym)
                        mid = 0.5 * (fs[d != 0].astype(np.float64) + sG[d != 0].astype(np.float64))
                        forced["scale_max_distance"] = max(forced["scale_max_distance"],
                                                           float(np.max(np.abs(pre - mid) / mid)))
                    sG = fs
                    if not sym and forced_zeros is not None:
                        fz = np.asarray(forced_zeros).astype(np.int64).reshape(m, ng)[:, G]
                        dz = np.abs(fz - zG.astype(np.int64))
                        forced["zero_mismatch"] += int((dz != 0).sum())
                        forced["zero_max_step"] = max(forced["zero_max_step"], int(dz.max()))
                        zG = fz.astype(np.uint16)
                scales[:, G] = sG
                if not sym:
                    zeros[:, G] = zG
            zc = None if sym else zeros[:, G]
            w = cur[:, j - b0] - E[:, b0:j] @ U[b0:j, j]      # this block's earlier columns
            q = _codes(w, scales[:, G], zc, bits, sym)
            if forced is not None:
                qf = np.asarray(forced_codes[:, j]).astype(q.dtype)
                diff = qf.astype(np.int64) != q.astype(np.int64)
                if diff.any():
                    sd = scales[diff, G].astype(np.float64)
                    zd = 0.0 if sym else zeros[diff, G].astype(np.float64)
                    tq = np.where(sd > 0, w[diff] / np.where(sd > 0, sd, 1.0), 0.0) + zd
                    lo = np.minimum(qf[diff].astype(np.float64), q[diff].astype(np.float64))
                    forced["count"] += int(diff.sum())
                    forced["max_distance"] = max(forced["max_distance"], float(np.max(np.abs(tq - (lo + 0.5)))))
                    forced["max_step"] = max(forced["max_step"], int(np.max(np.abs(qf[diff].astype(np.int64) - q[diff].astype(np.int64)))))
                q = qf
            codes_p[:, j] = q
            E[:, j] = (w - _value(scales[:, G], zc, q)) / U[j, j]
    res = _finish(codes_p, scales, perm, group_size, bits, zeros)
    if forced is not None:
        res["forced"] = forced
    return res


def gptq_unblocked(W: np.ndarray, U: np.ndarray, bits: int = 4, group_size: int = 128,
                   perm: Optional[np.ndarray] = None, scales_in: Optional[np.ndarray] = None,
                   sym: bool = True, zeros_in: Optional[np.ndarray] = None) -> dict:
    """The column loop as the method defines it, one column at a time ([GPTQ-P] "The GPTQ
    Algorithm", R1-R9): at a group's first column its scale (and zero) from the group's
    current values; the column's code; its error scaled by U_jj, e_j = (w_j - what_j) / U_jj;
    then every later column k moves by -e_j U_jk at once.  ``gptq`` computes the same
    result with the updates batched."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    Wp = W[:, perm].copy() if perm is not None else W.copy()
    g = _group_len(n, group_size)
    ng = n_groups(n, group_size)
    scales, zeros = _init_params(m, ng, scales_in, zeros_in, sym)
    codes_p = np.zeros((m, n), dtype=np.int8 if sym else np.uint8)
    for j in range(n):
        G = j // g
        if j % g == 0 and scales_in is None:
            sG, zG = _group_params(Wp[:, j:j + g], bits, sym)
            scales[:, G] = sG
            if not sym:
                zeros[:, G] = zG
        zc = None if sym else zeros[:, G]
        w = Wp[:, j]
        q = _codes(w, scales[:, G], zc, bits, sym)
        codes_p[:, j] = q
        e = (w - _value(scales[:, G], zc, q)) / U[j, j]
        Wp[:, j + 1:] -= np.outer(e, U[j, j + 1:])
    return _finish(codes_p, scales, perm, group_size, bits, zeros)


def rtn(W: np.ndarray, bits: int = 4, group_size: int = 128, scales_in: Optional[np.ndarray] = None,
        sym: bool = True, zeros_in: Optional[np.ndarray] = None) -> dict:
    """Round-to-nearest: scales from the original W per row ([GPT2-RE]) or per group of
    ``group_size`` consecutive columns ([MQM] "Group-wise Quantization"), then codes.
    ``sym=False``: the zero-point quantizer of A1-A4 (scale and zero per row and group)."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    g = _group_len(n, group_size)
    ng = n_groups(n, group_size)
    scales, zeros = _init_params(m, ng, scales_in, zeros_in, sym)
    if scales_in is None:
        for G in range(ng):
            sG, zG = _group_params(W[:, G * g:(G + 1) * g], bits, sym)
            scales[:, G] = sG
            if not sym:
                zeros[:, G] = zG
    codes = np.zeros((m, n), dtype=np.int8 if sym else np.uint8)
    for G in range(ng):
        zc = None if sym else zeros[:, G:G + 1]
        codes[:, G * g:(G + 1) * g] = _codes(W[:, G * g:(G + 1) * g], scales[:, G:G + 1], zc, bits, sym)
    What = dequant(codes, scales, group_size, out_dtype=np.float64, zeros=zeros)
    return {"codes": codes, "scales": scales, "zeros": zeros, "g_idx": None, "What": What,
            "bits": bits, "group_size": group_size}


def rtn_asym(W: np.ndarray, bits: int = 4, group_size: int = 128) -> dict:
    """``rtn`` with the zero-point quantizer (A1-A4)."""
    return rtn(W, bits, group_size, sym=False)


# ------------------------------------------------------------------ storage

def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, nibble = code + 8, even column in the low nibble (R10)."""
    c = np.asarray(codes, dtype=np.int16)
    m, n = c.shape
    if n % 2:
        raise ValueError("d_in must be even to pack two codes per byte")
    u = (c + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray, d_in: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], d_in), dtype=np.int8)
    codes[:, 0::2] = (p & 0x0F).astype(np.int16) - 8
    codes[:, 1::2] = (p >> 4).astype(np.int16) - 8
    return codes


def pack_uint4(codes: np.ndarray) -> np.ndarray:
    """Zero-point codes 0..15, two per byte, nibble = code, even column low (A4)."""
    c = np.asarray(codes, dtype=np.int16)
    m, n = c.shape
    if n % 2:
        raise ValueError("d_in must be even to pack two codes per byte")
    if c.size and (c.min() < 0 or c.max() > 15):
        raise ValueError("zero-point 4-bit codes lie in 0..15")
    u = c.astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_uint4(packed: np.ndarray, d_in: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    codes = np.empty((p.shape[0], d_in), dtype=np.uint8)
    codes[:, 0::2] = p & 0x0F
    codes[:, 1::2] = p >> 4
    return codes


def storage_bytes(d_out: int, d_in: int, group_size: int, zero_point: bool = False) -> int:
    """Bytes of the packed INT4 codes plus one float16 scale (and, with zero-points, one
    16-bit zero) per row and group ([GPTQ-P] "Group Quantization": 4 bits + 16 / group_size
    bits per weight for the scale, as many again for a zero)."""
    per_group = 4 if zero_point else 2
    return d_out * d_in // 2 + per_group * d_out * n_groups(d_in, group_size)


def dequant(codes: np.ndarray, scales: np.ndarray, group_size: int, g_idx: Optional[np.ndarray] = None,
            out_dtype=np.float64, zeros: Optional[np.ndarray] = None) -> np.ndarray:
    """What[r, c] = s[r, group(c)] * (code[r, c] - z[r, group(c)]) ([MQM] "Affine
    Quantization"; z = 0 without zero-points), exact in float64, then rounded once to
    ``out_dtype``."""
    codes = np.asarray(codes)
    m, n = codes.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64).reshape(m, -1)
    if group_size == 0:
        gi = np.zeros(n, dtype=np.int64)
    elif g_idx is not None:
        gi = np.asarray(g_idx, dtype=np.int64)
    else:
        gi = np.arange(n) // group_size
    q = codes.astype(np.float64)
    if zeros is not None:
        q = q - np.asarray(zeros, dtype=np.float64).reshape(m, -1)[:, gi]
    What = s[:, gi] * q
    return What.astype(out_dtype)


def dequant_asym(codes: np.ndarray, scales: np.ndarray, zeros: np.ndarray, group_size: int,
                 g_idx: Optional[np.ndarray] = None, out_dtype=np.float64) -> np.ndarray:
    """``dequant`` with zero-points."""
    return dequant(codes, scales, group_size, g_idx=g_idx, out_dtype=out_dtype, zeros=zeros)


# ------------------------------------------------------------------ activation-aware scaling

def channel_abs_mean(x_tiles: Union[np.ndarray, Iterable[np.ndarray]]) -> np.ndarray:
    """a_c = mean over all tokens of |X_tc| (W1), float64."""
    if isinstance(x_tiles, np.ndarray):
        x_tiles = [x_tiles]
    tot, ntok = None, 0
    for xt in x_tiles:
        x = np.abs(np.asarray(xt, dtype=np.float64))
        tot = x.sum(axis=0) if tot is None else tot + x.sum(axis=0)
        ntok += x.shape[0]
    return tot / ntok


def awq_scales(a: np.ndarray, alpha: float) -> np.ndarray:
    """s_c = a_c^alpha, 1 where a_c = 0 (W1)."""
    a = np.asarray(a, dtype=np.float64)
    return np.where(a > 0, np.power(np.where(a > 0, a, 1.0), alpha), 1.0)


def awq_search(W: np.ndarray, x_tiles, bits: int = 4, group_size: int = 128, n_alpha: int = 21,
               sym: bool = True) -> dict:
    """The grid search of W1 with RTN as the quantizer.  Returns the scores of every alpha,
    the winner's index, alpha and s, and the RTN result of W diag(s) (codes, scales, zeros)
    with What = its dequantization divided by s."""
    if isinstance(x_tiles, np.ndarray):
        x_tiles = [x_tiles]
    x_tiles = list(x_tiles)
    W = np.asarray(W, dtype=np.float64)
    a = channel_abs_mean(x_tiles)
    mses, results = [], []
    for k in range(n_alpha):
        alpha = k / (n_alpha - 1) if n_alpha > 1 else 0.0
        s = awq_scales(a, alpha)
        r = rtn(W * s[None, :], bits, group_size, sym=sym)
        What = r["What"] / s[None, :]
        mses.append(recon_mse(x_tiles, W, What))
        results.append((alpha, s, r, What))
    best = int(np.argmin(mses))                      # first minimum: ties to the smaller alpha
    alpha, s, r, What = results[best]
    return {"mse": np.array(mses), "best": best, "alpha": alpha, "s": s, "abs_mean": a,
            "codes": r["codes"], "scales": r["scales"], "zeros": r["zeros"], "What": What}


# ------------------------------------------------------------------ inference product

def quantized_matmul(X: np.ndarray, codes: np.ndarray, scales: np.ndarray, group_size: int,
                     zeros: Optional[np.ndarray] = None, g_idx: Optional[np.ndarray] = None) -> np.ndarray:
    """Y = X What^T in float64 (G1): X tokens x d_in, codes d_out x d_in with their scales
    (and zeros); What exact, the sum over d_in in float64."""
    What = dequant(codes, scales, group_size, g_idx=g_idx, out_dtype=np.float64, zeros=zeros)
    return np.asarray(X, dtype=np.float64) @ What.T


# ------------------------------------------------------------------ error measures

def recon_mse(x_tiles: Union[np.ndarray, Iterable[np.ndarray]], W: np.ndarray, What: np.ndarray,
              row_chunk: int = 2048) -> float:
    """Mean over tokens x outputs of (X W^T - X What^T)^2 ([GPT2-RE] step 5, R11)."""
    if isinstance(x_tiles, np.ndarray):
        x_tiles = [x_tiles]
    dW = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    total, ntok = 0.0, 0
    for xt in x_tiles:
        x = np.asarray(xt, dtype=np.float64)
        for r0 in range(0, x.shape[0], row_chunk):
            y = x[r0:r0 + row_chunk] @ dW.T
            total += float(np.sum(y * y))
        ntok += x.shape[0]
    return total / (ntok * dW.shape[0])


def recon_mse_trace(H_undamped: np.ndarray, n_tok: int, W: np.ndarray, What: np.ndarray) -> float:
    """Same quantity as ``recon_mse`` via ||X dW^T||^2 = tr(dW X^T X dW^T), X^T X = H / 2."""
    dW = np.asarray(W, dtype=np.float64) - np.asarray(What, dtype=np.float64)
    return float(np.einsum("ij,jk,ik->", dW, 0.5 * H_undamped, dW)) / (n_tok * dW.shape[0])


# ------------------------------------------------------------------ OBS reference (tiny sizes)

def direct_obs(W: np.ndarray, H: np.ndarray, bits: int, group_size: int = 0,
               scales_in: Optional[np.ndarray] = None, sym: bool = True,
               zeros_in: Optional[np.ndarray] = None) -> dict:
    """Sequential OBS in fixed left-to-right order, with no Cholesky factor at all.

    After column j is fixed at what_j, the still-free columns F = j+1.. move by the
    minimiser of the quadratic error restricted to F: delta_F = -(H_FF)^-1 H_Fj delta_j,
    delta_j = what_j - w_j ([GPTQ-P] "OBQ Foundation" and "Hessian-Based Weight Update"
    with R2).  Linear solves per step: tiny d_in only."""
    W = np.asarray(W, dtype=np.float64)
    m, n = W.shape
    g = _group_len(n, group_size)
    ng = n_groups(n, group_size)
    scales, zeros = _init_params(m, ng, scales_in, zeros_in, sym)
    codes = np.zeros((m, n), dtype=np.int8 if sym else np.uint8)
    Wc = W.copy()
    for j in range(n):
        G = j // g
        if j % g == 0 and scales_in is None:
            sG, zG = _group_params(Wc[:, j:j + g], bits, sym)
            scales[:, G] = sG
            if not sym:
                zeros[:, G] = zG
        zc = None if sym else zeros[:, G]
        q = _codes(Wc[:, j], scales[:, G], zc, bits, sym)
        codes[:, j] = q
        delta = _value(scales[:, G], zc, q) - Wc[:, j]
        Wc[:, j] += delta
        if j + 1 < n:
            F = slice(j + 1, n)
            step = np.linalg.solve(H[F, F], H[F, j])
            Wc[:, F] -= np.outer(delta, step)
    What = dequant(codes, scales, group_size, out_dtype=np.float64, zeros=zeros)
    return {"codes": codes, "scales": scales, "zeros": zeros, "What": What}


# ------------------------------------------------------------------ whole layer

def quantize_layer(W: np.ndarray, x_tiles, bits: int = 4, group_size: int = 128, block_size: int = 128,
                   damp: float = 0.01, act_order: bool = False, perm: Optional[np.ndarray] = None,
                   sym: bool = True) -> dict:
    """Hessian -> damping -> [act-order] -> U -> GPTQ, plus RTN and both MSEs on the same X.

    ``perm``: with act_order, a processing order decided elsewhere (the order is an integer
    decision taken on a floating-point diagonal; near-equal entries may be ordered either
    way, so a comparison can fix the order and check it separately)."""
    if isinstance(x_tiles, np.ndarray):
        x_tiles = [x_tiles]
    x_tiles = list(x_tiles)
    H = hessian(x_tiles)
    n_tok = sum(int(np.asarray(t).shape[0]) for t in x_tiles)
    Hd, lam = damp_hessian(H, damp)
    if act_order and perm is None:
        perm = act_order_perm(Hd)
    elif not act_order:
        perm = None
    Hp = Hd[np.ix_(perm, perm)] if perm is not None else Hd
    U = chol_inverse_upper(Hp)
    res = gptq(W, U, bits, group_size, block_size, perm=perm, sym=sym)
    r = rtn(W, bits, group_size, sym=sym)
    res.update({
        "H": H, "lambda": lam, "perm": perm, "U": U,
        "rtn": r,
        "gptq_mse": recon_mse(x_tiles, W, res["What"]),
        "rtn_mse": recon_mse(x_tiles, W, r["What"]),
        "n_tok": n_tok,
    })
    return res
