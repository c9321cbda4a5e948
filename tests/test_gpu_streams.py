"""Calls given a stream that is NOT torch's current stream.

The binding allocates outputs and temporaries (activation codes and scales,
the one-call linear's workspace) while the caller's stream is made current,
so torch's caching allocator ties them to the stream the kernels run on. This
test frees and reallocates memory on the current stream while the side
stream's kernels may still run, and checks the side stream's results against
the oracle.
"""
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _churn(nbytes, rounds=8):
    """Allocate and fill buffers of the temporaries' size on the current stream."""
    bufs = []
    for i in range(rounds):
        b = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        b.fill_(0x5A + i)
        bufs.append(b)
    return bufs


@pytest.mark.parametrize("kind", ["w8a8", "w8a8_pg", "w4a8", "token_group", "linear_ws"])
def test_side_stream_temporaries(kind):
    c = cider()
    M, N, K = 512, 1024, 2048
    x = inputs.activations(M, K, seed=81)
    w = inputs.weights(N, K, seed=81)
    xd, wd = dev(x), dev(w)
    gs = 128 if kind in ("w8a8_pg", "token_group") else 0
    bits = 4 if kind == "w4a8" else 8
    wq, sw = c.cider_quant_weight(wd, bits, gs)

    def call(stream=None):
        if kind in ("w8a8", "w8a8_pg"):
            return c.w8a8_linear(xd, wq, sw, gs, stream=stream)
        if kind == "w4a8":
            return c.w4a8_linear(xd, wq, sw, stream=stream)
        if kind == "token_group":
            return c.w8a8_linear_token_group(xd, wq, sw, gs, stream=stream)
        return c.cider_linear(xd, wq, sw, 8, 0, stream=stream)

    y_ref = call()                 # the same kernels on the current stream
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    assert side != torch.cuda.current_stream()
    outs = []
    for _ in range(4):   # several calls, each freeing its temporaries on return
        outs.append(call(side))
        _churn(M * K)          # may reuse freed memory only if it was tied to the side stream
    side.synchronize()
    torch.cuda.synchronize()
    for y in outs:
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), kind
    if kind == "w8a8":
        wqo, swo = oracle.quantize_weight(w, 8, 0)
        yo, _, _ = oracle.w8a8_linear(x, wqo, swo, 0)
        assert_y_close(y_ref.cpu().numpy(), yo, 1e-3, max_ulp=1, what=kind)
