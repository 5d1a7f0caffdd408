"""GPU parity of activation-aware channel scaling (pwq_channel_abs_mean, pwq_awq_search)
against the float64 oracle.

Channel means within one float32 ulp; every candidate's score within 1e-4 of the oracle's
(the GPU scores through its float32 H, the oracle over the tokens directly); the same winner
whenever the oracle's best and second-best scores differ by more than 1e-3; the winner's s
within 4 float32 ulps (double pow on both sides, float32 rounding on the GPU); its RTN codes
identical on >= 99.9 % with mismatches +-1 (W s is formed in float32 on the GPU)."""
import numpy as np
import pytest
import torch

import oracle as O
from post_weight_quantization_27_amd import synth
from test_gpu_parity import DEV, dev, dev_bf16, host, rand_w, code_agreement

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def pwq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_27_amd import pwq as P
    P.lib()
    return P


@pytest.mark.parametrize("N,n,xdt", [(1000, 200, "f32"), (4100, 768, "bf16"), (1, 33, "f32"), (2048, 1030, "bf16")])
def test_channel_abs_mean(pwq, N, n, xdt):
    rng = np.random.default_rng(N + n)
    Xf = rng.standard_normal((N, n)) * np.where(rng.random(n) < 0.05, 20.0, 1.0)
    if xdt == "bf16":
        bits = synth.f64_to_bf16_bits(Xf)
        Xd, X64 = dev_bf16(bits), synth.as_f64(bits, synth.BF16)
    else:
        X32 = Xf.astype(np.float32)
        Xd, X64 = dev(X32), X32.astype(np.float64)
    got = host(pwq.channel_abs_mean(Xd)).astype(np.float64)
    want = O.channel_abs_mean(X64)
    assert np.all(np.abs(got - want) <= 2.0 ** -23 * np.abs(want))


def test_channel_abs_mean_strided(pwq):
    rng = np.random.default_rng(96)
    big = rng.standard_normal((700, 300)).astype(np.float32)
    got = host(pwq.channel_abs_mean(dev(big)[:, :256])).astype(np.float64)
    want = O.channel_abs_mean(big[:, :256].astype(np.float64))
    assert np.all(np.abs(got - want) <= 2.0 ** -23 * np.abs(want))


def _run(pwq, W, X32, g, K, sym, bits=4):
    n = W.shape[1]
    Xd = dev(X32)
    H = torch.zeros((n, n), dtype=torch.float32, device=DEV)
    pwq.hessian_accumulate(Xd, H)
    a = pwq.channel_abs_mean(Xd)
    got = pwq.awq_search(dev(W), H, X32.shape[0], a, bits, g, K, zero_point=not sym,
                         want_packed=(bits == 4 and n % 2 == 0))
    want = O.awq_search(W, X32.astype(np.float64), bits, g, n_alpha=K, sym=sym)
    mse = host(got["mse"])
    assert np.all(np.abs(mse - want["mse"]) <= 1e-4 * want["mse"]), (mse, want["mse"])
    best = int(host(got["best"])[0])
    srt = np.sort(want["mse"])
    if len(srt) == 1 or srt[1] - srt[0] > 1e-3 * srt[0]:
        assert best == want["best"], (best, want["best"], want["mse"])
        s = host(got["s"]).astype(np.float64)
        assert np.all(np.abs(s - want["s"]) <= 4 * 2.0 ** -24 * want["s"])
        agree, maxd = code_agreement(host(got["codes"]), want["codes"])
        assert maxd <= 1 and agree >= 0.999, (agree, maxd)
        if bits == 4 and n % 2 == 0:
            pk = O.pack_int4 if sym else O.pack_uint4
            assert np.array_equal(host(got["packed"]), pk(host(got["codes"])))
    return best, want


@pytest.mark.parametrize("m,n,N,g,sym,wdt", [(96, 256, 1200, 128, True, np.float32), (64, 250, 900, 10, True, np.float32),
                                             (80, 512, 1500, 0, False, np.float16), (48, 384, 1000, 128, False, np.float32)])
def test_awq_search(pwq, m, n, N, g, sym, wdt):
    rng = np.random.default_rng(m * n + N)
    W = rand_w(rng, m, n, wdt)
    X = rng.standard_normal((N, n)).astype(np.float32)
    X[:, rng.choice(n, max(1, n // 50), replace=False)] *= 20
    X[:, 7] = 0.0                                            # a dead channel: s = 1
    best, want = _run(pwq, W, X, g, 11, sym)
    print(f"m={m} n={n} g={g} sym={sym}: best alpha index {best}, scores {np.round(want['mse'] / want['mse'][0], 4)}")


def test_awq_search_single_candidate_is_rtn(pwq):
    rng = np.random.default_rng(97)
    W = rand_w(rng, 64, 256)
    X = rng.standard_normal((600, 256)).astype(np.float32)
    Xd = dev(X)
    H = torch.zeros((256, 256), dtype=torch.float32, device=DEV)
    pwq.hessian_accumulate(Xd, H)
    got = pwq.awq_search(dev(W), H, 600, pwq.channel_abs_mean(Xd), 4, 128, 1)
    r = pwq.rtn_quantize(dev(W), 4, 128)
    assert torch.equal(got["codes"], r["codes"]) and torch.all(got["s"] == 1.0).item()


def test_awq_search_gpt2_layer(pwq):
    """The GPT-2-small c_fc layer (768 -> 3072) with its 8192 calibration tokens."""
    spec = synth.layer("gpt2_block", "h0.c_fc")
    W = synth.weight(spec)
    X = synth.x_full(spec)
    best, want = _run(pwq, W, X, spec.group_size, 21, True)
    print(f"c_fc: best alpha {want['alpha']:.2f}, RTN mse {want['mse'][0]:.5g} -> {want['mse'][want['best']]:.5g}")


@pytest.mark.parametrize("m,n,N,sym", [(4096, 4096, 1024, True), (4352, 4100, 768, False)])
def test_awq_search_split_route(pwq, m, n, N, sym):
    """Layers of at least 256 output tiles of 256 x 256 score the candidates with the split
    bfloat16 product over one triangle of H (ragged panels in the second case)."""
    rng = np.random.default_rng(m + n)
    W = rand_w(rng, m, n)
    X = rng.standard_normal((N, n)).astype(np.float32)
    X[:, rng.choice(n, n // 50, replace=False)] *= 20
    X[:, 7] = 0.0
    best, want = _run(pwq, W, X, 128, 4, sym)
    print(f"m={m} n={n}: best alpha index {best}, scores {np.round(want['mse'] / want['mse'][0], 4)}")
