"""The one-call linear (cider_linear): fp16 x -> quantization -> GEMM -> fp16 y.

Its outputs must equal, bit for bit, the two calls it stands for
(cider_quant_act then cider_w8a8_gemm / cider_w4a8_gemm), and meet the
oracle's per-channel bar (|y - o| <= 1e-3*|o| + 2^-14, at most one fp16 ulp;
per-group: 2e-3 plus the fp32 summation bound). The one-launch route
(per-channel, M <= 2: the GEMV kernel quantizes its activations itself) and
the workspace route are both covered, for int8 and packed int4 weights.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host, pg_sum_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

ONE_LAUNCH = [(1, 10240, 2560), (2, 2560, 10240), (2, 300, 1056), (2, 130, 32768), (1, 17, 32), (1, 64, 65536)]


def _two_calls(c, xd, wq, sw, bits, gs):
    """quant_act + GEMM, the GEMM with its own split-K workspace when it plans
    one (the one-call linear takes the same split, so the same bits)."""
    M, K = xd.shape
    N = wq.shape[0]
    xq, sa = c.cider_quant_act(xd, gs)
    need = c.cider_gemm_workspace_size(M, N, K, bits, gs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    if bits == 8:
        return host(c.cider_w8a8_gemm(xq, sa, wq, sw, gs, workspace=ws))
    return host(c.cider_w4a8_gemm(xq, sa, wq, sw, workspace=ws))


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("M,N,K", ONE_LAUNCH)
def test_one_launch_linear(M, N, K, bits):
    c = cider()
    assert c.cider_linear_workspace_size(M, N, K, bits, 0) == 0
    x = inputs.activations(M, K, seed=41)
    w = inputs.weights(N, K, seed=41)
    xd = dev(x)
    wq, sw = c.cider_quant_weight(dev(w), bits, 0)
    y = host(c.cider_linear(xd, wq, sw, bits, 0))
    assert np.array_equal(y.view(np.uint16), _two_calls(c, xd, wq, sw, bits, 0).view(np.uint16))
    wqo, swo = oracle.quantize_weight(w, bits, 0)
    yo = oracle.w8a8_linear(x, wqo, swo, 0)[0] if bits == 8 else oracle.w4a8_linear(x, wqo, swo)[0]
    assert_y_close(y, yo, 1e-3, max_ulp=1, what=f"linear{bits} {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,bits,gs", [(3, 300, 1056, 8, 0), (4, 130, 16384, 4, 0), (5, 200, 1024, 8, 0), (16, 300, 2560, 4, 0), (70, 260, 1152, 8, 64),
                                           (9, 130, 1024, 8, 128), (300, 650, 2560, 8, 0), (4, 100, 1024, 8, 128),
                                           (1024, 2560, 10240, 8, 128), (3000, 10248, 1024, 4, 0)])
def test_workspace_linear(M, N, K, bits, gs):
    c = cider()
    need = c.cider_linear_workspace_size(M, N, K, bits, gs)
    assert need >= M * K
    x = inputs.activations(M, K, seed=42)
    w = inputs.weights(N, K, seed=42)
    xd = dev(x)
    wq, sw = c.cider_quant_weight(dev(w), bits, gs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = host(c.cider_linear(xd, wq, sw, bits, gs, workspace=ws))
    assert np.array_equal(y.view(np.uint16), _two_calls(c, xd, wq, sw, bits, gs).view(np.uint16))
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, M - 1, np.random.default_rng(3).integers(0, M, 24)])
    wqo, swo = oracle.quantize_weight(w, bits, gs)
    if bits == 4:
        yo = oracle.w4a8_linear(x[rows], wqo, swo)[0]
        assert_y_close(y[rows], yo, 1e-3, max_ulp=1, what=f"linear4 {M}x{N}x{K}")
    elif gs == 0:
        yo = oracle.w8a8_linear(x[rows], wqo, swo, 0)[0]
        assert_y_close(y[rows], yo, 1e-3, max_ulp=1, what=f"linear8 {M}x{N}x{K}")
    else:
        yo, qo, sao = oracle.w8a8_linear(x[rows], wqo, swo, gs)
        e = pg_sum_bound(qo, sao, wqo, swo, gs, np.arange(len(rows)))
        assert_y_close(y[rows], yo, 2e-3, extra_atol=e, what=f"linear pg{gs} {M}x{N}x{K}")


def test_one_launch_special_rows():
    """A zero row gives zeros; rows of extreme magnitude quantize as the
    standalone quantizer does (same codes, same outputs)."""
    c = cider()
    K, N = 2560, 256
    rng = np.random.default_rng(43)
    x = (rng.standard_normal((4, K)) * 0.3).astype(np.float16)
    x[1] = 0
    x[2, :] = np.float16(6.0e-8)                     # subnormal fp16 row
    x[3, ::7] = np.float16(60000.0)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    xd = dev(x)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    y = host(c.cider_linear(xd, wq, sw, 8, 0))
    assert not y[1].any()
    assert np.array_equal(y.view(np.uint16), _two_calls(c, xd, wq, sw, 8, 0).view(np.uint16))


# bf16 x -> bf16 y (cider_linear_dt): both routes, int8 and int4 weights; bit
# for bit the two bf16 calls it stands for, and within one bf16 ulp of the
# oracle's exactly rounded value (per group: plus the fp32 summation bound)
@pytest.mark.parametrize("M,N,K,bits,gs", [(1, 10240, 2560, 8, 0), (2, 300, 1056, 8, 0), (1, 2560, 10240, 4, 0),
                                           (2, 130, 32768, 4, 0), (300, 650, 2560, 8, 0), (16, 300, 2560, 4, 0),
                                           (70, 260, 1152, 8, 64), (1024, 2560, 10240, 8, 128)])
def test_linear_bf16(M, N, K, bits, gs):
    from tests.test_gpu_bf16 import bf16_ulp_distance, bits as bf_bits, to_bf16_dev
    c = cider()
    xd = to_bf16_dev(inputs.activations(M, K, seed=43).astype(np.float32))
    w = inputs.weights(N, K, seed=43)
    wq, sw = c.cider_quant_weight(dev(w), bits, gs)
    y = bf_bits(c.cider_linear(xd, wq, sw, bits, gs))
    xq, sa = c.cider_quant_act(xd, gs)
    need = c.cider_gemm_workspace_size(M, N, K, bits, gs)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    if bits == 8:
        y2 = c.cider_w8a8_gemm(xq, sa, wq, sw, gs, workspace=ws, out_dtype=torch.bfloat16)
    else:
        y2 = c.cider_w4a8_gemm(xq, sa, wq, sw, workspace=ws, out_dtype=torch.bfloat16)
    assert np.array_equal(y, bf_bits(y2))
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 24)])
    wqo, swo = oracle.quantize_weight(w, bits, gs)
    xb = bf_bits(xd)[rows]
    if bits == 4:
        yo, qo, sao = oracle.w4a8_linear_bf16(xb, wqo, swo)
    else:
        yo, qo, sao = oracle.w8a8_linear_bf16(xb, wqo, swo, gs)
    if gs == 0:
        assert int(bf16_ulp_distance(y[rows], yo).max()) <= 1
    else:
        yv, ov = oracle.bf16_to_f32(y[rows]).astype(np.float64), oracle.bf16_to_f32(yo).astype(np.float64)
        e = pg_sum_bound(qo, sao, wqo, swo, gs, np.arange(len(rows)))
        assert np.all(np.abs(yv - ov) <= 2.0 ** -7 * np.abs(ov) + e + 2.0 ** -133), float(np.abs(yv - ov).max())
