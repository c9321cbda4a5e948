"""The full 28-layer Qwen3-VL-2B-shaped stack at seq 1024, every layer checked.

cider_stack_forward keeps only the last layer's intermediates, so the chain is
walked one layer at a time: layer l runs as a one-layer stack on the previous
layer's output, and each of its seven GEMMs (q, k, v, o, gate, up, down) is
held to the oracle fed the same fp16 inputs the GPU used, on sampled rows
(rows are independent through the stack: per-token quantization and row-wise
GEMMs). The one-shot 28-layer run must then reproduce the walked chain's
output bit for bit. Weight codes come from cider_quant_weight (held bit-exact
to the oracle elsewhere); the oracle dequantizes with the same codes and
scales.
"""
import numpy as np
import pytest

import oracle
from w8a8_online_quantized_amd import inputs
from tests.test_gpu_parity import assert_y_close, cider, dev, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ("q", "k", "v", "o", "gate", "up", "down")


def test_stack_28_layers_every_layer_on_sampled_rows():
    c = cider()
    M, dims, n_layers = 1024, (2048, 2048, 1024, 6144), 28
    hidden, q_dim, kv_dim, mlp_dim = dims
    shapes = {"q": (q_dim, hidden), "k": (kv_dim, hidden), "v": (kv_dim, hidden), "o": (hidden, q_dim),
              "gate": (mlp_dim, hidden), "up": (mlp_dim, hidden), "down": (hidden, mlp_dim)}
    layers, host_w = [], []
    for l in range(n_layers):
        L, H = {}, {}
        for name in NAMES:
            n, k = shapes[name]
            wq, ws = c.cider_quant_weight(dev(inputs.weights(n, k, seed=inputs.stack_weight_seed(l, name))), 8, 0)
            L[name] = (wq, ws)
            H[name] = (host(wq), host(ws))
        layers.append(c.fuse_stack_layer(L))
        host_w.append(H)
    rows = np.unique(np.r_[0, M - 1, np.random.default_rng(28).integers(0, M, 6)])
    x = dev(inputs.activations(M, hidden, seed=12))
    total, offs = c.cider_stack_workspace_layout(M, *dims)
    ws = torch.empty(total, dtype=torch.uint8, device="cuda")
    h = x
    for l in range(n_layers):
        y, _ = c.cider_stack_forward(h, [layers[l]], dims, workspace=ws)
        reg = {n: host(c.stack_region(ws, offs, n, M, *dims))[rows] for n in ("q", "k", "v", "o", "gate", "up")}
        inp = host(h)[rows]
        yl = host(y)[rows]
        H = host_w[l]
        for out, x16, wname in (("q", inp, "q"), ("k", inp, "k"), ("v", inp, "v"), ("o", reg["q"], "o"),
                                ("gate", reg["o"], "gate"), ("up", reg["o"], "up")):
            yo, _, _ = oracle.w8a8_linear(x16, H[wname][0], H[wname][1], 0)
            assert_y_close(reg[out], yo, 1e-3, max_ulp=1, what=f"layer {l} {out}")
        yo, _, _ = oracle.w8a8_linear(reg["up"], H["down"][0], H["down"][1], 0)
        assert_y_close(yl, yo, 1e-3, max_ulp=1, what=f"layer {l} down")
        assert np.isfinite(yl.astype(np.float32)).all(), f"layer {l}"
        h = y
    y_all, _ = c.cider_stack_forward(x, layers, dims)
    torch.cuda.synchronize()
    assert torch.equal(y_all.view(torch.int16), h.view(torch.int16))
