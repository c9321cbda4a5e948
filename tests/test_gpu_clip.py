"""Percentile-clipped weight scales (cider_quant_weight_clip) against
oracle.quantize_weight_clip: codes (or packed bytes) and scales bit for bit.

The threshold decides integer codes, so both sides take it in the same
precision (fp64 steps, fp32 result). Shapes cover per-channel rows from 16 to
131072 codes, per-group 64 / 128, int4, the percentiles 0, 50, 90, 99, 99.9
and 100 (= min-max, also checked against cider_quant_weight), rows with many
equal magnitudes and rows with outliers.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _weights(N, K, kind, seed):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return inputs.weights(N, K, seed=seed)
    if kind == "ties":          # few distinct magnitudes: many equal order statistics
        return (rng.integers(-4, 5, (N, K)) * 0.125).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)     # outliers
    idx = rng.integers(0, K, (N, 3))
    for r in range(N):
        w[r, idx[r]] = np.float16(2.5) * np.sign(rng.standard_normal(3)).astype(np.float16)
    return w


CASES = [(7, 16, 8, 0, 99.9, "normal"), (33, 1040, 8, 0, 99.9, "outliers"), (64, 2560, 8, 0, 99.9, "normal"),
         (16, 10240, 8, 0, 99.0, "outliers"), (8, 16384, 8, 0, 50.0, "normal"), (3, 131072, 8, 0, 99.9, "normal"),
         (40, 1024, 8, 64, 99.9, "outliers"), (40, 1024, 8, 128, 90.0, "normal"), (30, 2560, 4, 0, 99.9, "outliers"),
         (9, 256, 8, 0, 0.0, "normal"), (9, 256, 8, 0, 100.0, "normal"), (20, 2048, 8, 0, 99.9, "ties"),
         (20, 512, 8, 64, 37.5, "ties"), (12, 1024, 4, 0, 99.0, "ties")]


@pytest.mark.parametrize("N,K,bits,gs,p,kind", CASES)
def test_clip_codes_and_scales_bit_exact(N, K, bits, gs, p, kind):
    c = cider()
    w = _weights(N, K, kind, seed=N + K)
    q, s = c.cider_quant_weight_clip(dev(w), bits, gs, p)
    qo, so = oracle.quantize_weight_clip(w, bits, gs, p)
    assert np.array_equal(host(s), so), f"scales differ in {int((host(s) != so).sum())} groups"
    assert np.array_equal(host(q), qo), f"codes differ in {int((host(q) != qo).sum())} places"


@pytest.mark.parametrize("bits,gs", [(8, 0), (8, 64), (8, 128), (4, 0)])
def test_percentile_100_is_min_max(bits, gs):
    c = cider()
    w = _weights(50, 1024, "outliers", seed=7)
    q1, s1 = c.cider_quant_weight_clip(dev(w), bits, gs, 100.0)
    q0, s0 = c.cider_quant_weight(dev(w), bits, gs)
    assert np.array_equal(host(q1), host(q0)) and np.array_equal(host(s1), host(s0))


def test_clip_full_size_and_linear():
    """The 10240 x 2560 weight of the headline shape, then a W8A8 linear on
    the clipped codes against the oracle's linear on the oracle's codes."""
    c = cider()
    N, K = 10240, 2560
    w = inputs.weights(N, K, seed=3)
    q, s = c.cider_quant_weight_clip(dev(w), 8, 0, 99.9)
    qo, so = oracle.quantize_weight_clip(w, 8, 0, 99.9)
    assert np.array_equal(host(s), so) and np.array_equal(host(q), qo)
    x = inputs.activations(64, K, seed=3)
    y = host(c.w8a8_linear(dev(x), q, s, 0))
    yo, _, _ = oracle.w8a8_linear(x, qo, so, 0)
    assert_y_close(y, yo, 1e-3, max_ulp=1, what="clipped linear")
