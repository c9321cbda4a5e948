"""Per-channel / W4A8 store stage: bit-identical to the library's documented
fp32 arithmetic, fp16(fp32(fp32(acc) * s_a[m]) * s_w[n]), evaluated here in
numpy float32 on the oracle's codes, scales and exact integer accumulators.

The oracle itself rounds the fp64 product once (the kernel's two fp32
roundings stay within one fp16 ulp of it, checked elsewhere); this file pins
the kernel's own rounding sequence, so that a fused multiply-and-convert
(one rounding instead of two) anywhere in the store stages shows up. The
shapes reach every per-channel tile of the dispatch (GEMV, skinny and each
DMA tile) on sampled rows.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def fp32_two_step(acc, sa, sw):
    t = acc.astype(np.float32) * sa.astype(np.float32)[:, None]     # one fp32 rounding
    return (t * sw.astype(np.float32)[None, :]).astype(np.float16)   # fp32, then RNE fp16


def sampled(M, n=24):
    rng = np.random.default_rng(M)
    return np.unique(np.r_[0, M - 1, rng.integers(0, M, n)])


# (M, N, K): GEMV, skinny, 64x64, 64x160, 128x128, 128x256, 128x320, 256x320
PC_SHAPES = [(1, 10240, 2560), (9, 300, 2560), (70, 130, 1024), (1024, 2560, 10240), (2048, 2048, 1024),
             (1024, 6144, 2048), (1024, 10240, 2560), (4096, 10240, 2560), (300, 650, 1040)]


@pytest.mark.parametrize("M,N,K", PC_SHAPES)
def test_pc_store_stage_is_fp32_two_step(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=11)
    w = inputs.weights(N, K, seed=11)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0))
    rows = sampled(M)
    qo, sao = oracle.quantize_act(x[rows], 0)
    wqo, swo = oracle.quantize_weight(w, 8, 0)
    expect = fp32_two_step(oracle.int_dot(qo, wqo), sao, swo)
    got = y[rows]
    bad = got.view(np.uint16) != expect.view(np.uint16)
    assert not bad.any(), f"{int(bad.sum())} outputs differ from the fp32 two-step dequant"


@pytest.mark.parametrize("M,N,K", [(1, 10240, 2560), (7, 200, 512), (1024, 10240, 2560), (8192, 10240, 2560),
                                   (300, 650, 1056)])
def test_w4a8_store_stage_is_fp32_two_step(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=12)
    w = inputs.weights(N, K, seed=12)
    wp, sw = c.cider_quant_weight(dev(w), 4, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w4a8_gemm(xq, sa, wp, sw))
    rows = sampled(M)
    qo, sao = oracle.quantize_act(x[rows], 0)
    wpo, swo = oracle.quantize_weight(w, 4, 0)
    expect = fp32_two_step(oracle.int_dot(qo, oracle.unpack_int4(wpo)), sao, swo)
    bad = y[rows].view(np.uint16) != expect.view(np.uint16)
    assert not bad.any(), f"{int(bad.sum())} outputs differ from the fp32 two-step dequant"
