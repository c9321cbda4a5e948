"""Run-to-run determinism, one case per kernel family of the dispatch.

Every kernel here orders its arithmetic by hand (stage barriers, scheduling
barriers, the per-group scale ring, cross-wave reductions in wave order, the
split-K reductions in split order), so a repeated call on the same inputs must
reproduce its output bit for bit. Each case runs 20 repeats and stops at the
first mismatch; the comparison is on device, of the raw bit patterns.
"""
import numpy as np
import pytest

from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import cider, dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

REPEATS = 20

# (name, mode, M, N, K, group_size, use_workspace): the shape picks the family
FAMILIES = [
    ("256x320 persistent", "pc", 4096, 10240, 2560, 0, False),
    ("256x320 one round", "pc", 2048, 10240, 2560, 0, False),
    ("256x192 tile", "pc", 1024, 12288, 2048, 0, False),
    ("128x320 tile", "pc", 1024, 10240, 2560, 0, False),
    ("64x80 tile", "pc", 128, 10240, 2560, 0, False),
    ("64x128 tile", "pc", 1024, 2048, 6144, 0, False),
    ("64x64 four-stage tile", "pc", 1024, 2048, 2560, 0, False),
    ("64x160 tile", "pc", 64, 2560, 10240, 0, False),
    ("per-group gs128 ring", "pg", 1024, 2560, 10240, 128, False),
    ("per-group gs64 ring", "pg", 4096, 2560, 2048, 64, False),
    ("per-token x per-group", "tok", 1024, 2560, 10240, 128, False),
    ("W4A8", "w4", 1024, 10240, 2560, 0, False),
    ("skinny per-channel", "pc", 8, 2560, 10240, 0, False),
    ("skinny per-group", "pg", 8, 2560, 10240, 64, False),
    ("GEMV", "pc", 1, 10240, 2560, 0, False),
    ("GEMV W4A8", "w4", 2, 10240, 2560, 0, False),
    ("split-K int32 reduction", "pc", 256, 2560, 10240, 0, True),
    ("split-K fp32 reduction", "pg", 256, 2560, 10240, 128, True),
    ("split-K 64x160 eight ranges", "pg", 128, 2560, 10240, 64, True),
    ("decode MV", "mv", 1, 10240, 2560, 0, False),
    ("decode MV per-group", "mv", 2, 2560, 10240, 128, False),
]


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.element_size() == 2 else a.view(torch.int8),
                       b.view(torch.int16) if b.element_size() == 2 else b.view(torch.int8))


@pytest.mark.parametrize("name,mode,M,N,K,gs,ws", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_repeat_bit_identical(name, mode, M, N, K, gs, ws):
    c = cider()
    x = dev(inputs.activations(M, K, seed=71))
    w = dev(inputs.weights(N, K, seed=71))
    if mode == "mv":
        wq, sw = c.cider_quant_weight(w, 8, gs)
        call = lambda: c.cider_int8_mv(x, wq, sw, gs)   # noqa: E731
    else:
        bits = 4 if mode == "w4" else 8
        wq, sw = c.cider_quant_weight(w, bits, gs)
        xq, sa = c.cider_quant_act(x, 0 if mode in ("tok", "w4") else gs)
        wsb = c.cider_gemm_workspace_size(M, N, K, bits, gs) if ws else 0
        if ws:
            assert wsb > 0, f"{name}: expected a split-K plan"
        work = torch.empty(wsb, dtype=torch.uint8, device="cuda") if wsb else None
        if mode == "w4":
            call = lambda: c.cider_w4a8_gemm(xq, sa, wq, sw, workspace=work)   # noqa: E731
        elif mode == "tok":
            call = lambda: c.cider_w8a8_gemm_token_group(xq, sa, wq, sw, gs, workspace=work)   # noqa: E731
        else:
            call = lambda: c.cider_w8a8_gemm(xq, sa, wq, sw, gs, workspace=work)   # noqa: E731
    y0 = call()
    torch.cuda.synchronize()
    for i in range(REPEATS):
        y = call()
        torch.cuda.synchronize()
        assert _same(y, y0), f"{name}: repeat {i} differs from the first call"


@pytest.mark.parametrize("M,K,gs", [(4096, 2560, 0), (1024, 10240, 128), (3, 65536, 0), (512, 6144, 64)])
def test_quantizer_repeat_bit_identical(M, K, gs):
    c = cider()
    x = dev(inputs.activations(M, K, seed=72))
    q0, s0 = c.cider_quant_act(x, gs)
    torch.cuda.synchronize()
    for i in range(REPEATS):
        q, s = c.cider_quant_act(x, gs)
        torch.cuda.synchronize()
        assert torch.equal(q, q0) and torch.equal(s.view(torch.int32), s0.view(torch.int32)), f"repeat {i}"


def test_stack_repeat_bit_identical():
    c = cider()
    M, dims = 256, (512, 512, 256, 1536)
    hidden, q_dim, kv_dim, mlp_dim = dims
    shapes = {"q": (q_dim, hidden), "k": (kv_dim, hidden), "v": (kv_dim, hidden), "o": (hidden, q_dim),
              "gate": (mlp_dim, hidden), "up": (mlp_dim, hidden), "down": (hidden, mlp_dim)}
    layers = []
    for l in range(2):
        L = {n: c.cider_quant_weight(dev(inputs.weights(a, b, seed=inputs.stack_weight_seed(l, n))), 8, 0)
             for n, (a, b) in shapes.items()}
        layers.append(c.fuse_stack_layer(L))
    x = dev(inputs.activations(M, hidden, seed=73))
    y0, ws = c.cider_stack_forward(x, layers, dims)
    y0 = y0.clone()
    torch.cuda.synchronize()
    for i in range(REPEATS):
        y, _ = c.cider_stack_forward(x, layers, dims, workspace=ws)
        torch.cuda.synchronize()
        assert _same(y, y0), f"stack repeat {i}"
    assert np.isfinite(y0.float().cpu().numpy()).all()
