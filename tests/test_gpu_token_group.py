"""Per-token activations x per-group int8 weights (cider_w8a8_gemm_token_group)
against oracle.w8a8_linear_token_group, element by element.

The activation codes and their one-per-row scales must match the oracle bit for
bit; fp16 outputs must satisfy |y - o| <= 2e-3*|o| + e_sum + 2^-14, where o is
the oracle's exactly rounded output and e_sum = (G+17)*2^-24 * s_a[m] *
sum_g |acc_g*s_w[n,g]| bounds the fp32 group sum (at most G sequential fma
roundings in one wave, up to 15 more when the skinny kernel adds its waves'
partial sums, and the s_a product). The shapes reach the skinny kernel
(M <= 16) and every per-group tile of the dispatch, with ragged M, N and K
tails; the full-size cases check sampled rows.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def token_group_bound(qa, sa, qw, sw, gs):
    accg = oracle.int_dot_groups(qa, qw, gs).astype(np.float64)      # [G, rows, N]
    terms = np.abs(accg) * sw.T.astype(np.float64)[:, None, :]
    G = accg.shape[0]
    return (G + 17) * 2.0 ** -24 * sa.reshape(-1, 1).astype(np.float64) * terms.sum(axis=0)


def sampled(M, n=24, seed=0):
    rng = np.random.default_rng(seed + M)
    return np.unique(np.r_[0, M - 1, rng.integers(0, M, n)])


def _run(M, N, K, gs, seed, rows=None):
    c = cider()
    x = inputs.activations(M, K, seed=seed)
    w = inputs.weights(N, K, seed=seed)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    y = host(c.w8a8_linear_token_group(dev(x), wq, sw, gs))
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    assert np.array_equal(host(wq), wqo) and np.array_equal(host(sw), swo)
    rows = np.arange(M) if rows is None else rows
    yo, qo, sao = oracle.w8a8_linear_token_group(x[rows], wqo, swo, gs)
    e = token_group_bound(qo, sao, wqo, swo, gs)
    assert_y_close(y[rows], yo, 2e-3, extra_atol=e, what=f"token x pg{gs} {M}x{N}x{K}")
    return c, x, y


# (M, N, K, gs): skinny (M <= 16) with 4 / 8 / 16 waves, then the 64x64 and
# 128x128 per-group tiles, ragged tails
SMALL = [(1, 17, 128, 64), (3, 5, 128, 128), (16, 70, 2560, 64), (9, 300, 10240, 128), (1, 2560, 10240, 128),
         (33, 100, 1024, 128), (130, 300, 1152, 64), (520, 260, 2560, 128), (300, 650, 1280, 64),
         (257, 1000, 640, 128)]


@pytest.mark.parametrize("M,N,K,gs", SMALL)
def test_token_group_outputs(M, N, K, gs):
    _run(M, N, K, gs, seed=21)


# 128x160 and 128x128 tiles at both group sizes, ragged M and N (2498: scalar stores)
@pytest.mark.parametrize("M,N,K,gs", [(4000, 2500, 1280, 128), (2000, 2498, 1280, 128),
                                      (4000, 2498, 1280, 64), (2000, 2500, 1280, 64)])
def test_token_group_tiles_sampled(M, N, K, gs):
    _run(M, N, K, gs, seed=26, rows=sampled(M))


@pytest.mark.parametrize("M,N,K,gs", [(1024, 2560, 10240, 128), (4096, 2560, 10240, 128),
                                      (4096, 2560, 10240, 64), (128, 2560, 10240, 64)])
def test_token_group_full_size_sampled(M, N, K, gs):
    _run(M, N, K, gs, seed=22, rows=sampled(M))


def test_token_group_codes_and_scales_are_per_token():
    """The activation side of the linear is the per-channel quantizer: one
    scale per row, bit-identical codes."""
    c = cider()
    M, N, K, gs = 70, 130, 1024, 128
    x = inputs.activations(M, K, seed=23)
    xq, sa = c.cider_quant_act(dev(x), 0)
    qo, sao = oracle.quantize_act(x, 0)
    assert np.array_equal(host(xq), qo) and np.array_equal(host(sa), sao)


def test_token_group_special_rows():
    """Zero rows (scale 0) give zeros; a row that only overflows after the
    activation scale becomes +-inf exactly where the oracle's does."""
    c = cider()
    M, N, K, gs = 20, 64, 256, 64
    rng = np.random.default_rng(24)
    x = (rng.standard_normal((M, K)) * 0.5).astype(np.float16)
    x[3] = 0
    x[7] = np.float16(60000.0) * np.sign(rng.standard_normal(K)).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 2.0).astype(np.float16)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    y = host(c.w8a8_linear_token_group(dev(x), wq, sw, gs))
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    yo, qo, sao = oracle.w8a8_linear_token_group(x, wqo, swo, gs)
    assert not y[3].any()
    fin = np.isfinite(yo)
    assert np.array_equal(np.isfinite(y), fin)
    assert np.array_equal(np.sign(y[~fin]), np.sign(yo[~fin]))
    e = token_group_bound(qo, sao, wqo, swo, gs)
    assert_y_close(np.where(fin, y, 0), np.where(fin, yo, 0), 2e-3, extra_atol=np.where(fin, e, 0),
                   what="token x pg special rows")


def test_token_group_deterministic_and_stream_ordered():
    c = cider()
    M, N, K, gs = 300, 520, 2560, 128
    x = inputs.activations(M, K, seed=25)
    w = inputs.weights(N, K, seed=25)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y0 = host(c.cider_w8a8_gemm_token_group(xq, sa, wq, sw, gs))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1 = c.cider_w8a8_gemm_token_group(xq, sa, wq, sw, gs, stream=s)
    s.synchronize()
    assert np.array_equal(y0.view(np.uint16), host(y1).view(np.uint16))


# bf16 rows in, bf16 out (cider_w8a8_gemm_token_group_dt): the skinny kernel,
# the 64x64 / 128x128 / 128x160 tiles with ragged tails, and split-K (64x160
# in eight K ranges at M=128, 128x128 in three at M=1024)
@pytest.mark.parametrize("M,N,K,gs,split", [(3, 5, 128, 128, False), (16, 70, 2560, 64, False),
                                            (130, 300, 1152, 64, False), (520, 260, 2560, 128, False),
                                            (4000, 2500, 1280, 128, False), (2000, 2498, 1280, 64, False),
                                            (128, 2560, 10240, 128, True), (1024, 2560, 10240, 64, True)])
def test_token_group_bf16(M, N, K, gs, split):
    from tests.test_gpu_bf16 import bits, to_bf16_dev
    c = cider()
    xd = to_bf16_dev(inputs.activations(M, K, seed=23).astype(np.float32))
    w = inputs.weights(N, K, seed=23)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(xd, 0)
    ws = None
    if split:
        wsb = c.cider_gemm_workspace_size(M, N, K, 8, gs)
        assert wsb > 0
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    y = bits(c.cider_w8a8_gemm_token_group(xq, sa, wq, sw, gs, workspace=ws, out_dtype=torch.bfloat16))
    rows = np.arange(M) if M <= 520 else sampled(M)
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    yo, qo, sao = oracle.w8a8_linear_token_group_bf16(bits(xd)[rows], wqo, swo, gs)
    assert np.array_equal(host(xq)[rows], qo) and np.array_equal(host(sa)[rows], sao)
    e = token_group_bound(qo, sao, wqo, swo, gs)
    yv, ov = oracle.bf16_to_f32(y[rows]).astype(np.float64), oracle.bf16_to_f32(yo).astype(np.float64)
    # one bf16 ulp (at most 2^-7 |o|) plus the fp32 summation bound
    assert np.all(np.abs(yv - ov) <= 2.0 ** -7 * np.abs(ov) + e + 2.0 ** -133), float(np.abs(yv - ov).max())
