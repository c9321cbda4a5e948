"""Per-channel calls at K that is not a multiple of 16 (int8) or 32 (int4).

Rows then start at arbitrary byte offsets: the quantizer takes its
element-by-element path when K % 8 != 0, the GEMMs their general path for
unaligned rows. Codes, scales, packed bytes and int32 accumulators must match
the oracle bit for bit; fp16 / bf16 outputs within the per-channel bar
(1e-3 relative plus 2^-14, at most one ulp from the exactly rounded value).
Shapes span several 16 x 16 tiles with ragged M and N, and the last rows of a
buffer (whose fragments leave the buffer's range).
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("M,K", [(3, 1), (5, 2), (4, 3), (9, 7), (17, 15), (33, 40), (6, 100), (70, 2568),
                                 (2, 24), (130, 1000), (1, 16383)])
def test_quant_act_ragged(M, K):
    c = cider()
    x = inputs.activations(M, K, seed=111)
    q, s = c.cider_quant_act(dev(x), 0)
    qo, so = oracle.quantize_act(x, 0)
    assert np.array_equal(host(q), qo) and np.array_equal(host(s), so)
    xb = (x.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)   # bf16 patterns
    qb, sb = c.cider_quant_act(torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16), 0)
    qbo, sbo = oracle.quantize_rows_bf16(xb, 0, 127)
    assert np.array_equal(host(qb), qbo) and np.array_equal(host(sb), sbo[:, 0])


@pytest.mark.parametrize("N,K", [(3, 2), (5, 6), (17, 34), (9, 48), (40, 2570), (2, 8), (33, 1000)])
def test_quant_weight_int4_ragged(N, K):
    c = cider()
    w = inputs.weights(N, K, seed=112)
    p, s = c.cider_quant_weight(dev(w), 4, 0)
    po, so = oracle.quantize_weight(w, 4, 0)
    assert np.array_equal(host(p), po) and np.array_equal(host(s), so)
    q8, s8 = c.cider_quant_weight(dev(w), 8, 0)
    q8o, s8o = oracle.quantize_weight(w, 8, 0)
    assert np.array_equal(host(q8), q8o) and np.array_equal(host(s8), s8o)


ACC_CASES = [(1, 1, 1), (5, 9, 15), (17, 33, 40), (100, 300, 2568), (16, 16, 17), (3, 130, 1000),
             (33, 7, 127), (64, 80, 250)]


@pytest.mark.parametrize("M,N,K", ACC_CASES)
def test_acc_i32_ragged_bit_exact(M, N, K):
    c = cider()
    rng = np.random.default_rng(M * 13 + K)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    qa[0, :] = 127
    qw[-1, :] = -127                                   # extreme codes along the whole row
    acc = c.cider_gemm_acc_i32(0, dev(qa), dev(qw))
    assert np.array_equal(host(acc), oracle.int_dot(qa, qw))


@pytest.mark.parametrize("M,N,K", [(1, 5, 2), (4, 9, 34), (17, 40, 48), (100, 130, 2570), (3, 7, 6)])
def test_acc_i32_int4_ragged_bit_exact(M, N, K):
    c = cider()
    rng = np.random.default_rng(M * 17 + K)
    qa = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    q4 = rng.integers(-7, 8, size=(N, K)).astype(np.int8)
    acc = c.cider_gemm_acc_i32(1, dev(qa), dev(oracle.pack_int4(q4)))
    assert np.array_equal(host(acc), oracle.int_dot(qa, q4))


@pytest.mark.parametrize("M,N,K", [(1, 300, 1), (1, 100, 15), (5, 33, 40), (300, 520, 2568), (17, 2560, 200),
                                   (64, 10, 10007)])
def test_w8a8_ragged_outputs(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=113)
    w = inputs.weights(N, K, seed=113)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0))
    wqo, swo = oracle.quantize_weight(w, 8, 0)
    yo, qo, _ = oracle.w8a8_linear(x, wqo, swo, 0)
    assert np.array_equal(host(xq), qo) and np.array_equal(host(wq), wqo)
    assert_y_close(y, yo, 1e-3, max_ulp=1, what=f"ragged pc {M}x{N}x{K}")
    # the one-call linear (quantization through its workspace) gives the same bits
    yl = host(c.cider_linear(dev(x), wq, sw, 8, 0))
    assert np.array_equal(yl.view(np.uint16), y.view(np.uint16))
    # bf16 output: the same fp32 values rounded to bf16
    yb = c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16)
    ybf = host(yb.view(torch.int16)).view(np.uint16)
    ref = oracle.dequant_bf16(oracle.int_dot(qo, wqo), host(sa), swo)
    diff = np.abs(oracle.bf16_to_f32(ybf).astype(np.float64) - oracle.bf16_to_f32(ref).astype(np.float64))
    assert np.all(diff <= 2.0 ** -7 * np.abs(oracle.bf16_to_f32(ref).astype(np.float64)) + 2.0 ** -126)


@pytest.mark.parametrize("M,N,K", [(1, 70, 2), (3, 40, 34), (20, 33, 48), (130, 260, 1002), (2, 5000, 2570)])
def test_w4a8_ragged_outputs(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=114)
    w = inputs.weights(N, K, seed=114)
    wp, sw = c.cider_quant_weight(dev(w), 4, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w4a8_gemm(xq, sa, wp, sw))
    wpo, swo = oracle.quantize_weight(w, 4, 0)
    assert np.array_equal(host(wp), wpo)
    yo, _, _ = oracle.w4a8_linear(x, wpo, swo)
    assert_y_close(y, yo, 1e-3, max_ulp=1, what=f"ragged w4a8 {M}x{N}x{K}")
    yl = host(c.cider_linear(dev(x), wp, sw, 4, 0))
    assert np.array_equal(yl.view(np.uint16), y.view(np.uint16))
