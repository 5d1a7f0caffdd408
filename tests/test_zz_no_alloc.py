"""The allocation-free product (pwq_quantized_matmul_noalloc) against the product with a
caller workspace (pwq_quantized_matmul): same kernels, so the outputs must be identical, on
consecutive calls whose sizes shrink (the scratch array keeps the previous call's sums)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def pwq():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from post_weight_quantization_27_amd import pwq as P
    P.lib()
    return P


def _inputs(rng, T, n, m, g, zp):
    X = torch.from_numpy(rng.standard_normal((T, n)).astype(np.float16)).to(DEV)
    packed = torch.from_numpy(rng.integers(0, 256, (m, n // 2), dtype=np.uint8)).to(DEV)
    ng = 1 if g == 0 else n // g
    sc = (rng.uniform(0.5, 2.0, (m, ng)) * 0.003).astype(np.float16)
    scales = torch.from_numpy(sc.view(np.int16)).to(DEV).view(torch.float16)
    zeros = torch.from_numpy(rng.integers(0, 16, (m, ng)).astype(np.int16)).to(DEV) if zp else None
    return X, packed, scales, zeros


@pytest.mark.parametrize("zp,ydt", [(False, torch.float16), (True, torch.float32)])
def test_noalloc_matches_workspace_product(pwq, zp, ydt):
    rng = np.random.default_rng(91 + int(zp))
    # first call: 8 column splits over 8192 inputs; second: smaller in every dimension, with
    # 2 splits, so its sums land where the first call's were
    for T, n, m, g in ((16, 8192, 4096, 128), (3, 2048, 1000, 0 if zp else 256)):
        X, packed, scales, zeros = _inputs(rng, T, n, m, g, zp)
        want = pwq.quantized_matmul(X, packed, scales, g, zeros=zeros, out_dtype=ydt)
        got = torch.full((T, m), float("nan"), dtype=ydt, device=DEV)
        pwq.quantized_matmul_noalloc(X, packed, scales, got, g, zeros=zeros)
        torch.cuda.synchronize()
        assert torch.equal(got, want), (T, n, m, g)


def test_noalloc_rejects_more_than_its_scratch(pwq):
    rng = np.random.default_rng(93)
    X, packed, scales, _ = _inputs(rng, 64, 28672, 64, 128, False)
    out = torch.empty((64, 64), dtype=torch.float16, device=DEV)
    # 28 splits x 64 tokens x 64 rows fit; the same shape with 8192 rows does not
    pwq.quantized_matmul_noalloc(X, packed, scales, out, 128)
    torch.cuda.synchronize()
    assert torch.equal(out, pwq.quantized_matmul(X, packed, scales, 128))
    big = pwq.lib().pwq_quantized_matmul_workspace_size(64, 28672, 8192)
    assert big > (32 << 20)
    st = pwq.lib().pwq_quantized_matmul_noalloc(X.data_ptr(), 1, 64, 28672, 28672, packed.data_ptr(),
                                                scales.data_ptr(), None, 8192, 128, out.data_ptr(), 1, 8192, None)
    assert st == pwq.PWQ_EWORKSPACE
