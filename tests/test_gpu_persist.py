"""The persistent per-channel kernel (256 x 320 tiles, more than one round of
tiles, K % 128 == 0, N % 8 == 0) against the oracle, with int8 weights and
with packed int4 weights (W4A8).

Its seams are what these shapes aim at: blocks that walk different numbers of
tiles (tile counts that are not a multiple of 256), tiles cut by the M and N
edges, stage counts per tile that are odd, even and one (the buffer of a
tile's first stage alternates, and with one stage the last stage is also the
first), and fp16 and bf16 outputs. Every column of the sampled rows is
checked (the last tile-row and the ragged column tiles included): within one
ulp of the oracle's exactly rounded value, and bit-identical to the kernel's
documented fp32 two-step fp(fp32(fp32(acc) * s_a) * s_w).
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def tiles_256x320(M, N):
    return -(-M // 256) * -(-N // 320)


# (M, N, K): tile counts 512, 396, 341, 396; stages per tile 20, 8, 3, 1
SHAPES = [(4096, 10240, 2560), (3000, 10248, 1024), (2600, 9608, 384), (3000, 10248, 128)]


def rows_for(M, seed):
    rng = np.random.default_rng(seed)
    last = (M - 1) // 256 * 256   # first row of the last tile-row
    return np.unique(np.r_[0, 255, 256, last, M - 1, rng.integers(0, M, 10), rng.integers(last, M, 4)])


def two_step(acc, sa, sw):
    return (acc.astype(np.float32) * sa.astype(np.float32)[:, None]) * sw.astype(np.float32)[None, :]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_persist_fp16(M, N, K):
    assert tiles_256x320(M, N) > 256 and K % 128 == 0 and N % 8 == 0
    c = cider()
    x = inputs.activations(M, K, seed=81)
    w = inputs.weights(N, K, seed=81)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = c.cider_w8a8_gemm(xq, sa, wq, sw, 0)
    rows = rows_for(M, M + N + K)
    qo, sao = oracle.quantize_act(x[rows], 0)
    wqo, swo = oracle.quantize_weight(w, 8, 0)
    acc = oracle.int_dot(qo, wqo)
    yh = host(y)[rows]
    assert_y_close(yh, oracle.dequant_per_channel(acc, sao, swo), 1e-3, max_ulp=1, what=f"persist {M}x{N}x{K}")
    expect = two_step(acc, sao, swo).astype(np.float16)
    assert np.array_equal(yh.view(np.uint16), expect.view(np.uint16))


@pytest.mark.parametrize("M,N,K", SHAPES[1:3])
def test_persist_bf16(M, N, K):
    c = cider()
    x = inputs.activations(M, K, seed=82)
    w = inputs.weights(N, K, seed=82)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = rows_for(M, M + N)
    qo, sao = oracle.quantize_act(x[rows], 0)
    wqo, swo = oracle.quantize_weight(w, 8, 0)
    acc = oracle.int_dot(qo, wqo)
    yb = y.view(torch.int16).cpu().numpy().view(np.uint16)[rows]
    yo = oracle.dequant_bf16(acc, sao, swo)
    d = np.abs(yb.astype(np.int32) - yo.astype(np.int32))
    assert int(d.max()) <= 1, "bf16 output more than one ulp from the oracle"
    assert np.array_equal(yb, oracle.f64_to_bf16(two_step(acc, sao, swo).astype(np.float64)))


def test_persist_repeat_and_neighbours_untouched():
    """20 repeats bit-identical, and nothing written outside y (guard rows
    around it in one allocation stay as they were)."""
    c = cider()
    M, N, K = 3000, 10248, 1024
    x = dev(inputs.activations(M, K, seed=83))
    w = dev(inputs.weights(N, K, seed=83))
    wq, sw = c.cider_quant_weight(w, 8, 0)
    xq, sa = c.cider_quant_act(x, 0)
    buf = torch.full(((M + 2) * N,), 12345, dtype=torch.int16, device="cuda")
    y = buf[N:(M + 1) * N].view(torch.float16).view(M, N)
    c.cider_w8a8_gemm(xq, sa, wq, sw, 0, y=y)
    torch.cuda.synchronize()
    y0 = y.clone()
    for i in range(20):
        c.cider_w8a8_gemm(xq, sa, wq, sw, 0, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"repeat {i}"
    assert bool((buf[:N] == 12345).all()) and bool((buf[(M + 1) * N:] == 12345).all())


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_persist_w4a8(M, N, K):
    """Packed int4 weights: sampled rows within one ulp of the oracle's W4A8
    linear, and the whole output bit-identical to the int8 kernel run on the
    unpacked codes."""
    c = cider()
    x = inputs.activations(M, K, seed=84)
    w = inputs.weights(N, K, seed=84)
    wp, sw = c.cider_quant_weight(dev(w), 4, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    y = host(c.cider_w4a8_gemm(xq, sa, wp, sw))
    wpo, swo = oracle.quantize_weight(w, 4, 0)
    assert np.array_equal(host(wp), wpo)
    rows = rows_for(M, M + N + K + 4)
    yo, _, _ = oracle.w4a8_linear(x[rows], wpo, swo)
    assert_y_close(y[rows], yo, 1e-3, max_ulp=1, what=f"persist w4a8 {M}x{N}x{K}")
    y8 = host(c.cider_w8a8_gemm(xq, sa, dev(oracle.unpack_int4(wpo)), sw, 0))
    assert np.array_equal(y.view(np.uint16), y8.view(np.uint16))


def test_persist_w4a8_bf16_repeat_and_neighbours_untouched():
    """bf16 output of the W4A8 persistent kernel: bit-identical to the int8
    kernel on the unpacked codes, 20 repeats bit-identical, and nothing
    written outside y."""
    c = cider()
    M, N, K = 3000, 10248, 1024
    x = dev(inputs.activations(M, K, seed=85))
    w = inputs.weights(N, K, seed=85)
    wp, sw = c.cider_quant_weight(dev(w), 4, 0)
    xq, sa = c.cider_quant_act(x, 0)
    buf = torch.full(((M + 2) * N,), 12345, dtype=torch.int16, device="cuda")
    y = buf[N:(M + 1) * N].view(torch.bfloat16).view(M, N)
    c.cider_w4a8_gemm(xq, sa, wp, sw, y=y)
    torch.cuda.synchronize()
    y8 = c.cider_w8a8_gemm(xq, sa, dev(oracle.unpack_int4(host(wp))), sw, 0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y8.view(torch.int16))
    y0 = y.clone()
    for i in range(20):
        c.cider_w4a8_gemm(xq, sa, wp, sw, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y0.view(torch.int16)), f"repeat {i}"
    assert bool((buf[:N] == 12345).all()) and bool((buf[(M + 1) * N:] == 12345).all())
