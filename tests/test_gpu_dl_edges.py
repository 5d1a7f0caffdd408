"""Parity of the large-tile products (256 x 256 and 128 x 128 tiles) on their edges.

The far updates of the factor, its near updates (with the next diagonal factor in the same
launch) and the GPTQ trailing products run on the large-tile engines once a launch has
enough tiles: the deepest, on 256 x 256 tiles, as six bfloat16 products of their operands'
three-piece splits (the split route), the others on the direct-load float32 engine, 128 x 128
tiles below.  The full-size layers have dimensions that are multiples of 256; these cases
add what those do not reach:

* the factor at n = 12000: push tiles with a ragged last column block (rows of the split
  pieces zero past the matrix, outputs discarded by the epilogue), diagonal syrk tiles (the
  per-element triangle test), and a first super-block 736 deep (not a multiple of 128);
* GPTQ with 12000 rows and 4608 inputs: ragged last row tile in the trailing products, and
  launches on the split route and on the float32 engines within one layer;
* GPTQ with 9000 rows and 4700 inputs: a split-route product whose columns end in a ragged
  tile (3676 of them), a ragged last block and group (92 columns); symmetric, and with
  zero-points (codes compared as grid indices code - Z, the zeros within one).

Inputs are seeded; the float64 references are the oracle's (``oracle.chol_inverse_upper`` up
to 8192 inputs, the same textbook route through torch.linalg on the device past that, as in
the full-size tests; ``oracle.gptq`` on sampled rows, including rows of the ragged tile).
"""
import numpy as np
import pytest
import torch

import oracle as O
from test_gpu_fullsize import DEV, factor64_device, host, log, rel_frob_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pwq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_27_amd import pwq as P
    P.lib()
    return P


def damped_hessian64(n, n_tok, seed):
    g = torch.Generator(device=DEV).manual_seed(seed)
    H = torch.zeros((n, n), dtype=torch.float64, device=DEV)
    for t0 in range(0, n_tok, 4096):
        x = torch.randn((min(4096, n_tok - t0), n), generator=g, device=DEV, dtype=torch.float32)
        x = x.to(torch.bfloat16).to(torch.float64)
        H.addmm_(x.t(), x)
    H.mul_(2.0)
    H.diagonal().add_(0.01 * float(torch.diagonal(H).mean()))
    return H


def test_factor_large_tiles_ragged(pwq):
    n = 12000
    H32 = damped_hessian64(n, 2 * n, 71).to(torch.float32)
    U, info = pwq.chol_inverse_upper(H32)
    assert int(host(info)[0]) == 0
    U64 = factor64_device(H32.double())
    rf = rel_frob_dev(U, U64)
    # every row block, including the ragged last one and the block rows of the 736-deep
    # first super-block
    worst = max(rel_frob_dev(U[r0:r0 + 256], U64[r0:r0 + 256]) for r0 in range(0, n, 256))
    log(f"factor n={n}: U rel-Frob {rf:.3g}, worst 256-row block {worst:.3g}")
    assert torch.count_nonzero(torch.tril(U, -1)) == 0
    assert bool(torch.all(torch.diagonal(U) > 0))
    assert rf <= 1e-5 and worst <= 2e-5


def test_gptq_large_tiles_ragged_rows(pwq):
    m, n, g, B = 12000, 4608, 128, 128
    H64 = damped_hessian64(n, 2 * n, 72)
    U64 = O.chol_inverse_upper(host(H64))
    del H64
    Ud = torch.from_numpy(U64.astype(np.float32)).to(DEV)
    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(73)
    W = (rng.standard_t(4.0, size=(m, n)) * 0.0106).astype(np.float16)
    res = pwq.gptq_quantize_layer(torch.from_numpy(W).to(DEV), Ud, info, 4, g, B)
    rows = np.sort(np.concatenate([rng.choice(11776, 96, replace=False), np.arange(11968, 12000)]))
    want = O.gptq(W[rows], U64, 4, g, B)
    codes = host(res["codes"])[rows]
    sc = host(res["scales"])[rows]
    d = np.abs(codes.astype(np.int16) - want["codes"].astype(np.int16))
    agree = float(np.mean(d == 0))
    rep = O.gptq(W[rows], U64, 4, g, B, forced_codes=codes, forced_scales=sc)
    f = rep["forced"]
    log(f"gptq {m}x{n}: codes agree {agree:.6f} (max diff {d.max()}), replay {f}")
    assert d.max() <= 1 and agree >= 0.999
    assert f["max_step"] <= 1 and f["max_distance"] <= 1e-3 and f["count"] <= 1e-3 * codes.size
    assert f["scale_max_ulp"] <= 1 and f["scale_max_distance"] <= 1e-4


def test_gptq_split_route_ragged_columns(pwq):
    m, n, g, B = 9000, 4700, 128, 128
    H64 = damped_hessian64(n, 2 * n, 74)
    U64 = O.chol_inverse_upper(host(H64))
    del H64
    Ud = torch.from_numpy(U64.astype(np.float32)).to(DEV)
    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(75)
    W = (rng.standard_t(4.0, size=(m, n)) * 0.0106).astype(np.float16)
    res = pwq.gptq_quantize_layer(torch.from_numpy(W).to(DEV), Ud, info, 4, g, B)
    # rows of every row tile, the ragged last one (8960 .. 8999) among them
    rows = np.sort(np.concatenate([rng.choice(8960, 96, replace=False), np.arange(8968, 9000)]))
    want = O.gptq(W[rows], U64, 4, g, B)
    codes = host(res["codes"])[rows]
    sc = host(res["scales"])[rows]
    d = np.abs(codes.astype(np.int16) - want["codes"].astype(np.int16))
    agree = float(np.mean(d == 0))
    rep = O.gptq(W[rows], U64, 4, g, B, forced_codes=codes, forced_scales=sc)
    f = rep["forced"]
    log(f"gptq {m}x{n}: codes agree {agree:.6f} (max diff {d.max()}), replay {f}")
    assert d.max() <= 1 and agree >= 0.999
    assert f["max_step"] <= 1 and f["max_distance"] <= 1e-3 and f["count"] <= 1e-3 * codes.size
    assert f["scale_max_ulp"] <= 1 and f["scale_max_distance"] <= 1e-4


def test_gptq_zp_split_route_ragged_columns(pwq):
    m, n, g, B = 9000, 4700, 128, 128
    H64 = damped_hessian64(n, 2 * n, 76)
    U64 = O.chol_inverse_upper(host(H64))
    del H64
    Ud = torch.from_numpy(U64.astype(np.float32)).to(DEV)
    info = torch.zeros(1, dtype=torch.int32, device=DEV)
    rng = np.random.default_rng(77)
    W = (rng.standard_t(4.0, size=(m, n)) * 0.0106).astype(np.float16)
    res = pwq.gptq_quantize_layer_zp(torch.from_numpy(W).to(DEV), Ud, info, 4, g, B)
    rows = np.sort(np.concatenate([rng.choice(8960, 96, replace=False), np.arange(8968, 9000)]))
    want = O.gptq(W[rows], U64, 4, g, B, sym=False)
    gi = np.arange(n) // g
    z = host(res["zeros"])[rows].astype(np.int32)
    zw = want["zeros"].astype(np.int32)
    # a zero one off shifts its whole group: compare the grid indices code - Z
    got = host(res["codes"])[rows].astype(np.int32) - z[:, gi]
    ref = want["codes"].astype(np.int32) - zw[:, gi]
    d = np.abs(got - ref)
    agree = float(np.mean(d == 0))
    log(f"gptq zero-point {m}x{n}: grid indices agree {agree:.6f} (max diff {d.max()}), "
        f"zeros equal {float(np.mean(z == zw)):.5f}")
    assert d.max() <= 1 and agree >= 0.999
    assert np.abs(z - zw).max() <= 1 and np.mean(z == zw) >= 0.99
