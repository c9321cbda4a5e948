"""Same-input projections as one GEMM (cider_w8a8_gemm_split) against the
oracle, part by part.

Each part's output must satisfy the per-channel bar against oracle.w8a8_linear
of that part's weights on the shared activation codes (|y - o| <= 1e-3*|o| +
2^-14, at most one fp16 ulp), and must equal, bit for bit, what
cider_w8a8_gemm computes for the part alone. The shapes reach the per-part
small-M route (M <= 16) and the fused DMA tiles, with 2, 3 and 4 parts and
part boundaries inside tiles.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = [(1, 256, (48, 16, 80)), (5, 1024, (256, 128, 128)), (16, 2560, (640, 320)),
         (70, 256, (256, 128, 128)), (300, 640, (16, 32, 48, 64)), (257, 1040, (336, 48, 176)),
         (1024, 2048, (2048, 1024, 1024)), (1024, 2048, (6144, 6144))]


@pytest.mark.parametrize("M,K,parts", CASES)
def test_split_parts_match_oracle_and_unfused(M, K, parts):
    c = cider()
    x = inputs.activations(M, K, seed=31)
    ws = [inputs.weights(n, K, seed=31 + i) for i, n in enumerate(parts)]
    q = [c.cider_quant_weight(dev(w), 8, 0) for w in ws]
    wcat = torch.cat([a for a, _ in q])
    scat = torch.cat([b for _, b in q])
    xq, sa = c.cider_quant_act(dev(x), 0)
    ys = [host(y) for y in c.cider_w8a8_gemm_split(xq, sa, wcat, scat, parts)]
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 24)])
    for i, (w, (wq, sw)) in enumerate(zip(ws, q)):
        alone = host(c.cider_w8a8_gemm(xq, sa, wq, sw, 0))
        assert np.array_equal(ys[i].view(np.uint16), alone.view(np.uint16)), f"part {i} differs from its own GEMM"
        wqo, swo = oracle.quantize_weight(w, 8, 0)
        yo, _, _ = oracle.w8a8_linear(x[rows], wqo, swo, 0)
        assert_y_close(ys[i][rows], yo, 1e-3, max_ulp=1, what=f"split part {i} {M}x{parts}x{K}")


def test_split_leaves_memory_outside_the_parts_alone():
    c = cider()
    M, K, parts = 40, 512, (64, 32)
    x = inputs.activations(M, K, seed=32)
    w = inputs.weights(sum(parts), K, seed=32)
    wq, sw = c.cider_quant_weight(dev(w), 8, 0)
    xq, sa = c.cider_quant_act(dev(x), 0)
    buf = torch.full((3 * M * 128,), -7.0, dtype=torch.float16, device="cuda")
    y0 = buf[M * 128:M * 128 + M * 64].view(M, 64)
    y1 = buf[2 * M * 128:2 * M * 128 + M * 32].view(M, 32)
    c.cider_w8a8_gemm_split(xq, sa, wq, sw, parts, ys=[y0, y1])
    b = host(buf)
    untouched = np.ones(b.size, bool)
    untouched[M * 128:M * 128 + M * 64] = False
    untouched[2 * M * 128:2 * M * 128 + M * 32] = False
    assert np.all(b[untouched] == -7.0)


@pytest.mark.parametrize("M,K,parts", [(5, 1024, (256, 128, 128)), (300, 640, (16, 32, 48, 64)),
                                       (1024, 2048, (2048, 1024, 1024))])
def test_split_bf16_parts_match_their_own_bf16_gemm(M, K, parts):
    """bf16 outputs (cider_w8a8_gemm_split_dt): every part equals, bit for bit,
    the bf16 GEMM of that part alone, and lies within one bf16 ulp of the
    oracle's exactly rounded value."""
    from tests.test_gpu_bf16 import bf16_ulp_distance, bits
    c = cider()
    x = inputs.activations(M, K, seed=32)
    ws = [inputs.weights(n, K, seed=32 + i) for i, n in enumerate(parts)]
    q = [c.cider_quant_weight(dev(w), 8, 0) for w in ws]
    wcat = torch.cat([a for a, _ in q])
    scat = torch.cat([b for _, b in q])
    xq, sa = c.cider_quant_act(dev(x), 0)
    ys = [bits(y) for y in c.cider_w8a8_gemm_split(xq, sa, wcat, scat, parts, out_dtype=torch.bfloat16)]
    rows = np.arange(M) if M <= 300 else np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 24)])
    qo = host(xq)[rows]
    so = host(sa)[rows]
    for i, (w, (wq, sw)) in enumerate(zip(ws, q)):
        alone = bits(c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16))
        assert np.array_equal(ys[i], alone), f"part {i} differs from its own bf16 GEMM"
        yo = oracle.dequant_bf16(oracle.int_dot(qo, host(wq)), so, host(sw))
        assert int(bf16_ulp_distance(ys[i][rows], yo).max()) <= 1, i
