"""cider_w8a8_gemm_noalloc (the GEMM for callers that cannot allocate: split-K
scratch in the library's own device array) against cider_w8a8_gemm_ex with
a caller workspace, through the C ABI: bit-identical outputs on two calls in
a row, the second one smaller, for per-channel and per-group shapes that
split K and one that does not; the first output also within the oracle bar
on sampled rows; and every split plan of a shape sweep fits the scratch.
"""
import ctypes

import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host, pg_sum_bound

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def S():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _operands(c, M, N, K, gs, seed):
    x = inputs.activations(M, K, seed=seed)
    w = inputs.weights(N, K, seed=seed)
    wq, sw = c.cider_quant_weight(dev(w), 8, gs)
    xq, sa = c.cider_quant_act(dev(x), gs)
    return x, w, xq, sa, wq, sw


def _both(c, L, xq, sa, wq, sw, M, N, K, gs):
    """(y from the no-allocation call, y from the workspace call)."""
    y_na = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = L.cider_w8a8_gemm_noalloc(P(xq), P(sa), P(wq), P(sw), M, N, K, gs, P(y_na), 0, S())
    assert st == 0, c.status_string(st)
    need = L.cider_gemm_workspace_size(M, N, K, 8, gs)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda") if need else None
    y_ws = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = L.cider_w8a8_gemm_ex(P(xq), P(sa), P(wq), P(sw), M, N, K, gs, P(y_ws), 0, P(ws), need, S())
    assert st == 0, c.status_string(st)
    torch.cuda.synchronize()
    return y_na, y_ws, need


# (first shape, second smaller shape, group size): each pair splits K (the
# scratch holds the first call's slabs when the second call runs)
PAIRS = [((1024, 2560, 10240), (256, 2560, 10240), 0),
         ((1024, 2560, 10240), (128, 2560, 10240), 128),
         ((512, 2560, 10240), (256, 2560, 10240), 64),
         ((1024, 2560, 10240), (300, 650, 8192), 0)]


@pytest.mark.parametrize("first,second,gs", PAIRS)
def test_noalloc_matches_workspace_call(first, second, gs):
    c = cider()
    L = c.lib()
    outs = []
    for i, (M, N, K) in enumerate((first, second)):
        g = gs if K % max(gs, 1) == 0 else 0
        x, w, xq, sa, wq, sw = _operands(c, M, N, K, g, seed=101 + i)
        y_na, y_ws, need = _both(c, L, xq, sa, wq, sw, M, N, K, g)
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), (M, N, K, g, need)
        outs.append((x, w, M, N, K, g, y_na))
    # the first call's output against the oracle on sampled rows
    x, w, M, N, K, g, y = outs[0]
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(M).integers(0, M, 16)])
    wqo, swo = oracle.quantize_weight(w, 8, g)
    yo, qo, sao = oracle.w8a8_linear(x[rows], wqo, swo, g)
    if g == 0:
        assert_y_close(host(y)[rows], yo, 1e-3, max_ulp=1, what=f"noalloc {M}x{N}x{K}")
    else:
        e = pg_sum_bound(qo, sao, wqo, swo, g, np.arange(len(rows)))
        assert_y_close(host(y)[rows], yo, 2e-3, extra_atol=e, what=f"noalloc pg{g} {M}x{N}x{K}")


def test_noalloc_bf16_and_unsplit():
    c = cider()
    L = c.lib()
    M, N, K = 128, 2560, 10240
    _, _, xq, sa, wq, sw = _operands(c, M, N, K, 0, seed=105)
    y_na = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    assert L.cider_w8a8_gemm_noalloc(P(xq), P(sa), P(wq), P(sw), M, N, K, 0, P(y_na), 1, S()) == 0
    y_ref = c.cider_w8a8_gemm(xq, sa, wq, sw, 0, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16))
    M, N, K = 4096, 10240, 2560        # no split: no scratch used
    assert L.cider_gemm_workspace_size(M, N, K, 8, 0) == 0
    _, _, xq, sa, wq, sw = _operands(c, M, N, K, 0, seed=106)
    y_na, y_ws, _ = _both(c, L, xq, sa, wq, sw, M, N, K, 0)
    assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16))


def test_noalloc_scratch_covers_every_plan():
    c = cider()
    L = c.lib()
    limit = c.NOALLOC_SCRATCH_BYTES
    # no current plan needs more than the array; the check still guards it:
    # every planned shape in a sweep stays within the limit
    for M in (64, 128, 256, 512, 1024, 2048):
        for N, K in ((2560, 10240), (2048, 6144), (4096, 16384), (10240, 8192)):
            for gs in (0, 64, 128):
                assert L.cider_gemm_workspace_size(M, N, K, 8, gs) <= limit, (M, N, K, gs)
    assert c.status_string(c.CIDER_ERROR_SCRATCH_LIMIT)
