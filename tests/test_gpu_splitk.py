"""Split-K (cider_w8a8_gemm_ex / cider_w4a8_gemm_ex with a workspace) for
medium M with long K: outputs bit-identical to the unsplit GEMM (the int32
partial sums are exact) and within the per-channel bar of the oracle on
sampled rows; ragged N takes the scalar reduction; bf16 output and W4A8 too;
a workspace reused by a second, smaller call stays correct.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SHAPES = [(128, 2560, 10240), (256, 2560, 10240), (1024, 2560, 10240), (300, 650, 8192), (130, 2048, 6144),
          (64, 4096, 16384)]


def _ws(c, M, N, K, bits=8):
    need = c.cider_gemm_workspace_size(M, N, K, bits, 0)
    assert need > 0, f"{M}x{N}x{K} was expected to split"
    return torch.empty(need, dtype=torch.uint8, device="cuda")


def _rows(M):
    return np.arange(M) if M <= 300 else np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 24)])


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_split_k_bit_identical_and_oracle(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=61)
    w = inputs.weights(N, K, seed=61)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y0 = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0))
    y1 = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0, workspace=_ws(c, M, N, K)))
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))
    rows = _rows(M)
    wqo, swo = oracle.quantize_weight(w, 8, 0)
    yo, _, _ = oracle.w8a8_linear(x[rows], wqo, swo, 0)
    assert_y_close(y1[rows], yo, 1e-3, max_ulp=1, what=f"split-K {M}x{N}x{K}")


def test_split_k_bf16_and_w4a8():
    c = cider()
    M, N, K = 128, 2560, 10240
    x = inputs.activations(M, K, seed=62)
    w = inputs.weights(N, K, seed=62)
    xq, sa = c.cider_quant_act(dev(x), 0)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    b0 = c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16)
    b1 = c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16, workspace=_ws(c, M, N, K))
    torch.cuda.synchronize()
    assert torch.equal(b0.view(torch.int16), b1.view(torch.int16))
    wp, sw4 = c.cider_quant_weight(dev(w), 4, 0)
    y0 = host(c.cider_w4a8_gemm(xq, sa, wp, sw4))
    y1 = host(c.cider_w4a8_gemm(xq, sa, wp, sw4, workspace=_ws(c, M, N, K, bits=4)))
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))
    wpo, swo = oracle.quantize_weight(w, 4, 0)
    yo, _, _ = oracle.w4a8_linear(x, wpo, swo)
    assert_y_close(y1, yo, 1e-3, max_ulp=1, what="split-K W4A8")


def test_split_k_workspace_reuse_and_linear():
    c = cider()
    big = (1024, 2560, 10240)
    small = (130, 2048, 6144)
    ws = _ws(c, *big)
    assert ws.numel() >= c.cider_gemm_workspace_size(*small, 8, 0)
    for (M, N, K) in (big, small):
        x = inputs.activations(M, K, seed=63)
        w = inputs.weights(N, K, seed=63)
        xq, sa = c.cider_quant_act(dev(x), 0)
        wq, sw = c.cider_quant_weight(dev(w), 8, 0)
        y0 = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0))
        y1 = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0, workspace=ws))
        assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16)), (M, N, K)
        # the one-call linear sizes and uses the same slabs after its codes
        need = c.cider_linear_workspace_size(M, N, K, 8, 0)
        assert need > M * K
        y2 = host(c.cider_linear(dev(x), wq, sw, 8, 0))
        assert np.array_equal(y0.view(np.uint16), y2.view(np.uint16)), (M, N, K)


# ---------------------------------------------------------------- per-group split-K (fp32 partial sums)
from tests.test_gpu_parity import pg_sum_bound  # noqa: E402
from tests.test_gpu_token_group import token_group_bound  # noqa: E402

# 64x160 tiles with 8 K ranges (at most 32 tiles, K >= 8192; ragged M, N and
# a last range of two stages at K = 8320), 64x64 with 4 / 2 ranges (M = 256,
# M = 500 at K = 4096), 128x128 with 4 (161..320 tiles of 64x64 and
# K >= 8192: M = 500 at K = 8192, ragged M and N) and with 3 (M=1024; ragged
# at gs 64) and, for gs 128, 128x160 with 2 (M=2048; ragged M, N = 2498:
# scalar stores in the reduction)
PG = [(128, 2560, 10240, 128), (128, 2560, 10240, 64), (130, 650, 8192, 128), (64, 1024, 16384, 64),
      (100, 1990, 8320, 128), (100, 1990, 8320, 64), (256, 2560, 10240, 64), (500, 2000, 4096, 128),
      (500, 2000, 8192, 128), (500, 2000, 8192, 64),
      (1024, 2560, 10240, 128), (1000, 2500, 8192, 64), (2048, 2560, 10240, 128), (1800, 2498, 4096, 128)]


def _rows(M):
    if M <= 256:
        return np.arange(M)
    return np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 32)])


@pytest.mark.parametrize("M,N,K,gs", PG)
def test_split_k_per_group(M, N, K, gs):
    c = cider()
    need = c.cider_gemm_workspace_size(M, N, K, 8, gs)
    assert need > 0, f"{M}x{N}x{K} gs{gs} was expected to split"
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    x = inputs.activations(M, K, seed=64)
    w = inputs.weights(N, K, seed=64)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(dev(x), gs)
    y = host(c.cider_w8a8_gemm(xq, sa, wq, sw, gs, workspace=ws))
    rows = _rows(M)
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    yo, qo, sao = oracle.w8a8_linear(x[rows], wqo, swo, gs)
    e = pg_sum_bound(qo, sao, wqo, swo, gs, np.arange(len(rows)))
    assert_y_close(y[rows], yo, 2e-3, extra_atol=e, what=f"split-K pg{gs} {M}x{N}x{K}")
    # deterministic: the same bits again
    y2 = host(c.cider_w8a8_gemm(xq, sa, wq, sw, gs, workspace=ws))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16))


@pytest.mark.parametrize("M,gs", [(128, 128), (128, 64), (1024, 64), (2048, 128)])
def test_split_k_token_group(M, gs):
    c = cider()
    N, K = 2560, 10240
    ws = torch.empty(c.cider_gemm_workspace_size(M, N, K, 8, gs), dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    x = inputs.activations(M, K, seed=65)
    w = inputs.weights(N, K, seed=65)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w8a8_gemm_token_group(xq, sa, wq, sw, gs, workspace=ws))
    rows = _rows(M)
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    yo, qo, sao = oracle.w8a8_linear_token_group(x[rows], wqo, swo, gs)
    e = token_group_bound(qo, sao, wqo, swo, gs)
    assert_y_close(y[rows], yo, 2e-3, extra_atol=e, what=f"split-K token x pg{gs} M={M}")


def test_split_k_per_group_bf16():
    c = cider()
    M, N, K, gs = 128, 2560, 10240, 128
    ws = torch.empty(c.cider_gemm_workspace_size(M, N, K, 8, gs), dtype=torch.uint8, device="cuda")
    x32 = inputs.activations(M, K, seed=66).astype(np.float32)
    xd = torch.from_numpy(x32).to(torch.bfloat16).cuda()
    w = inputs.weights(N, K, seed=66)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(xd, gs)
    y = c.cider_w8a8_gemm(xq, sa, wq, sw, gs, out_dtype=torch.bfloat16, workspace=ws)
    torch.cuda.synchronize()
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)
    xb = xd.view(torch.int16).cpu().numpy().view(np.uint16)
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    yo, qo, sao = oracle.w8a8_linear_bf16(xb, wqo, swo, gs)
    yv, ov = oracle.bf16_to_f32(yb).astype(np.float64), oracle.bf16_to_f32(yo).astype(np.float64)
    e = pg_sum_bound(qo, sao, wqo, swo, gs, np.arange(M))
    assert np.all(np.abs(yv - ov) <= 2.0 ** -7 * np.abs(ov) + e + 2.0 ** -133)
