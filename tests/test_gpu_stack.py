"""The chained linear-stack driver (cider_stack_forward) against the oracle.

Every GEMM of the last layer is checked against the oracle fed the same fp16
input the GPU used (read back from the driver's workspace), and the layer
hand-off is checked by determinism: the input the last layer of an L-layer
run reads equals the output of an (L-1)-layer run, bit for bit.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def make_layers(c, n_layers, dims, seed0=0):
    hidden, q_dim, kv_dim, mlp_dim = dims
    shapes = {"q": (q_dim, hidden), "k": (kv_dim, hidden), "v": (kv_dim, hidden), "o": (hidden, q_dim),
              "gate": (mlp_dim, hidden), "up": (mlp_dim, hidden), "down": (hidden, mlp_dim)}
    layers, host_w = [], []
    for l in range(n_layers):
        L, H = {}, {}
        for name, (N, K) in shapes.items():
            w = inputs.weights(N, K, seed=seed0 + inputs.stack_weight_seed(l, name))
            wq, ws = c.cider_quant_weight(dev(w), 8, 0)
            L[name] = (wq, ws)
            H[name] = oracle.quantize_weight(w, 8, 0)
        layers.append(L)
        host_w.append(H)
    return layers, host_w


def ref_linear(x16, wq_ws):
    wq, ws = wq_ws
    y, _, _ = oracle.w8a8_linear(x16, wq, ws, 0)
    return y


def check_last_layer(c, x, ws, offs, y, M, dims, H, rows, inp):
    hidden, q_dim, kv_dim, mlp_dim = dims
    reg = {n: host(c.stack_region(ws, offs, n, M, hidden, q_dim, kv_dim, mlp_dim))[rows]
           for n in ("q", "k", "v", "o", "gate", "up")}
    yh = host(y)[rows]
    checks = [("q", inp, "q"), ("k", inp, "k"), ("v", inp, "v"), ("o", reg["q"], "o"),
              ("gate", reg["o"], "gate"), ("up", reg["o"], "up")]
    for out_name, x16, wname in checks:
        assert_y_close(reg[out_name], ref_linear(x16, H[wname]), 1e-3, max_ulp=1, what=f"stack {out_name}")
    assert_y_close(yh, ref_linear(reg["up"], H["down"]), 1e-3, max_ulp=1, what="stack down")


@pytest.mark.parametrize("M,dims,n_layers", [(70, (256, 256, 128, 512), 1), (70, (256, 256, 128, 512), 3),
                                             (1024, (2048, 2048, 1024, 6144), 2)])
def test_stack_chain(M, dims, n_layers):
    c = cider()
    hidden = dims[0]
    x = inputs.activations(M, hidden, seed=9)
    layers, H = make_layers(c, n_layers, dims)
    total, offs = c.cider_stack_workspace_layout(M, *dims)
    y, ws = c.cider_stack_forward(dev(x), layers, dims)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 128 else np.unique(np.r_[0, M - 1, np.random.default_rng(1).integers(0, M, 40)])
    if n_layers == 1:
        inp = x[rows]
    else:
        # input of the last layer: the output of the first n_layers-1 layers
        y_prev, _ = c.cider_stack_forward(dev(x), layers[:-1], dims)
        h = host(c.stack_region(ws, offs, "h", M, *dims))
        assert np.array_equal(h.view(np.uint16), host(y_prev).view(np.uint16))
        inp = h[rows]
    check_last_layer(c, x, ws, offs, y, M, dims, H[-1], rows, inp)


@pytest.mark.parametrize("M,dims", [(70, (256, 256, 128, 512)), (9, (256, 256, 128, 512)),
                                    (1024, (2048, 2048, 1024, 6144))])
def test_stack_fused_projections_are_bit_identical(M, dims):
    """Adjacent q/k/v and gate/up weights run as one GEMM each; every output
    and intermediate equals the unfused run bit for bit."""
    c = cider()
    x = inputs.activations(M, dims[0], seed=10)
    layers, _ = make_layers(c, 2, dims, seed0=5)
    fused = [c.fuse_stack_layer(L) for L in layers]
    y0, ws0 = c.cider_stack_forward(dev(x), layers, dims)
    y1, ws1 = c.cider_stack_forward(dev(x), fused, dims)
    torch.cuda.synchronize()
    assert np.array_equal(host(y0).view(np.uint16), host(y1).view(np.uint16))
    _, offs = c.cider_stack_workspace_layout(M, *dims)
    for n in ("q", "k", "v", "o", "gate", "up"):
        a = host(c.stack_region(ws0, offs, n, M, *dims))
        b = host(c.stack_region(ws1, offs, n, M, *dims))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), n



@pytest.mark.parametrize("M,dims,n_layers", [(70, (256, 256, 128, 512), 2), (9, (256, 256, 128, 512), 1),
                                             (1024, (2048, 2048, 1024, 6144), 1)])
def test_stack_bf16(M, dims, n_layers):
    """The bf16 chain (cider_stack_forward_dt): every GEMM of the last layer
    within one bf16 ulp of the oracle fed the same bf16 input (read back from
    the workspace), fused and unfused projections bit-identical, and the
    layer hand-off as for fp16."""
    from tests.test_gpu_bf16 import bf16_ulp_distance, bits, to_bf16_dev
    c = cider()
    hidden, q_dim, kv_dim, mlp_dim = dims
    xd = to_bf16_dev(inputs.activations(M, hidden, seed=11).astype(np.float32))
    layers, H = make_layers(c, n_layers, dims, seed0=7)
    y, ws = c.cider_stack_forward(xd, layers, dims)
    fused = [c.fuse_stack_layer(L) for L in layers]
    y1, ws1 = c.cider_stack_forward(xd, fused, dims)
    assert np.array_equal(bits(y), bits(y1))
    _, offs = c.cider_stack_workspace_layout(M, *dims)
    reg = {n: bits(c.stack_region(ws, offs, n, M, *dims, dtype=torch.bfloat16))
           for n in ("q", "k", "v", "o", "gate", "up")}
    for n in reg:
        assert np.array_equal(reg[n], bits(c.stack_region(ws1, offs, n, M, *dims, dtype=torch.bfloat16))), n
    rows = np.arange(M) if M <= 128 else np.unique(np.r_[0, M - 1, np.random.default_rng(2).integers(0, M, 32)])
    if n_layers == 1:
        inp = bits(xd)
    else:
        y_prev, _ = c.cider_stack_forward(xd, layers[:-1], dims)
        inp = bits(c.stack_region(ws, offs, "h", M, *dims, dtype=torch.bfloat16))
        assert np.array_equal(inp, bits(y_prev))
    Hl = H[-1]
    checks = [("q", inp, "q"), ("k", inp, "k"), ("v", inp, "v"), ("o", reg["q"], "o"),
              ("gate", reg["o"], "gate"), ("up", reg["o"], "up")]
    for out_name, xin, wname in checks:
        yo, _, _ = oracle.w8a8_linear_bf16(xin[rows], *Hl[wname], 0)
        assert int(bf16_ulp_distance(reg[out_name][rows], yo).max()) <= 1, out_name
    yo, _, _ = oracle.w8a8_linear_bf16(reg["up"][rows], *Hl["down"], 0)
    assert int(bf16_ulp_distance(bits(y)[rows], yo).max()) <= 1, "down"
