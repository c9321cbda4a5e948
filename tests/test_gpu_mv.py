"""Decode MV (cider_int8_mv: fp16 activations, int8 weights dequantized on the
fly) against the CPU oracle.

The oracle rounds the exact value once; the kernel sums in fp32 along a fixed
tree (per lane K/32 codes in v_dot2 pairs, then 8 lanes, then 4 waves), so each
output is held to |y - o| <= 1e-3*|o| + (K/32 + 24)*2^-24*sum_k|x*q*s| + 2^-14
(fp16 rounding, the fp32 summation bound of that tree, the fp16 subnormal
step). Shapes: the README's decode shapes [N=10240, K=2560] and [N=2560,
K=10240] at M = 1, per-channel and per-group, plus ragged N, several M <= 4,
special values and the full range of int8 codes; both the LDS-staged
activation path and the cache-read path (M * K * 2 > 64 KiB) are exercised.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def mv_bound(x, q, s, gs):
    K = x.shape[1]
    G = 1 if gs == 0 else K // gs
    sk = np.repeat(np.asarray(s, np.float64).reshape(q.shape[0], G), K // G, axis=1)
    terms = np.abs(x.astype(np.float64)) @ (np.abs(q.astype(np.float64)) * sk).T
    return (K / 32 + 24) * 2.0 ** -24 * terms


def check(y, x, q, s, gs, what):
    o = oracle.int8_mv(x, q, s, gs).astype(np.float64)
    y64 = y.astype(np.float64)
    tol = 1e-3 * np.abs(o) + mv_bound(x, q, s, gs) + 2.0 ** -14
    err = np.abs(y64 - o)
    bad = err > tol
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs out of tolerance, worst {float((err - tol).max())}"


CASES = [(1, 10240, 2560, 0), (1, 2560, 10240, 0), (1, 2560, 10240, 128), (1, 2560, 10240, 64),
         (1, 10240, 2560, 128), (2, 300, 1040, 0), (3, 77, 256, 64), (4, 1030, 2560, 128), (4, 5, 16, 0),
         (1, 9, 128, 128), (2, 4097, 4096, 64),
         # activations too large for the LDS-staged path (M * K * 2 > 64 KiB): cache-read path
         (4, 300, 10240, 0), (3, 130, 16384, 128)]


@pytest.mark.parametrize("M,N,K,gs", CASES)
def test_int8_mv(M, N, K, gs):
    c = cider()
    x = inputs.activations(M, K, seed=21 + M)
    w = inputs.weights(N, K, seed=22)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    y = host(c.cider_int8_mv(dev(x), wq, sw, gs))
    wqo, swo = oracle.quantize_weight(w, 8, gs)
    assert np.array_equal(host(wq), wqo)
    check(y, x, wqo, swo, gs, f"mv {M}x{N}x{K} gs{gs}")


def test_int8_mv_extreme_codes_and_values():
    """Codes at +-127 and -127..127 sweeps, activations at fp16 extremes that
    keep the outputs finite (large and subnormal magnitudes, signed zeros)."""
    c = cider()
    rng = np.random.default_rng(5)
    M, N, K = 2, 64, 512
    q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    q[0, :] = 127
    q[1, :] = -127
    q[2, :] = np.arange(K) % 255 - 127
    x = (rng.standard_normal((M, K)) * 2.0 ** rng.integers(-24, 4, size=(M, K))).astype(np.float16)
    x[0, :8] = np.float16(-0.0)
    x[1, :4] = np.float16(60000.0)
    x[1, 4:8] = np.float16(-60000.0)
    for gs in (0, 64, 128):
        G = 1 if gs == 0 else K // gs
        s = (np.abs(rng.standard_normal((N, G))) * 1e-4 + 1e-6).astype(np.float32)
        s_arg = s[:, 0] if gs == 0 else s
        y = host(c.cider_int8_mv(dev(x), dev(q), dev(np.ascontiguousarray(s_arg)), gs))
        check(y, x, q, s_arg, gs, f"extreme gs{gs}")


def test_int8_mv_deterministic_and_stream_ordered():
    c = cider()
    x = inputs.activations(1, 2560, seed=3)
    w = inputs.weights(10240, 2560, seed=4)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xd = dev(x)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ys = [c.cider_int8_mv(xd, wq, sw, 0, stream=s) for _ in range(3)]
    s.synchronize()
    a = [host(y).view(np.uint16) for y in ys]
    assert np.array_equal(a[0], a[1]) and np.array_equal(a[0], a[2])
