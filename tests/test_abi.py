"""The C-ABI library loads, exports every symbol include/cider.h declares, and
rejects bad arguments before touching HIP (no GPU needed)."""
import ctypes

import pytest

from w8a8_online_quantized_amd import cider

L = None


def setup_module(_):
    global L
    L = cider.lib()


def test_exports_every_header_symbol():
    names = cider.header_entry_points()
    assert set(names) == set(cider.SIGNATURES), names
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    for s in range(4):
        assert L.cider_status_string(s)
    assert b"unknown" in L.cider_status_string(99)
    assert cider.cider_version() >= 100


# A fake, 16-byte aligned, non-null device address: argument checks that fail
# return before any HIP call, so it is never dereferenced.
P = ctypes.c_void_p(1 << 20)
MIS = ctypes.c_void_p((1 << 20) + 8)
NULL = None
INV = cider.CIDER_ERROR_INVALID_VALUE


@pytest.mark.parametrize("M,K,gs", [(-1, 64, 0), (4, 0, 0), (4, -8, 0), (4, 96, 64),
                                    (4, 128, 32), (4, 133120 + 128, 0), (4, 100, 64)])
def test_quant_act_rejects_bad_sizes(M, K, gs):
    assert L.cider_quant_act(P, M, K, gs, P, P, NULL) == INV


def test_quant_act_rejects_null_and_misaligned():
    assert L.cider_quant_act(NULL, 4, 64, 0, P, P, NULL) == INV
    assert L.cider_quant_act(P, 4, 64, 0, NULL, P, NULL) == INV
    assert L.cider_quant_act(P, 4, 64, 0, P, NULL, NULL) == INV
    assert L.cider_quant_act(MIS, 4, 64, 0, P, P, NULL) == INV
    assert L.cider_quant_act(P, 4, 64, 0, MIS, P, NULL) == INV


def test_empty_work_is_success_without_pointers():
    assert L.cider_quant_act(NULL, 0, 64, 0, NULL, NULL, NULL) == 0
    assert L.cider_quant_weight(NULL, 0, 64, 8, 0, NULL, NULL, NULL) == 0
    assert L.cider_w8a8_gemm(NULL, NULL, NULL, NULL, 0, 16, 64, 0, NULL, NULL) == 0
    assert L.cider_w8a8_gemm(NULL, NULL, NULL, NULL, 16, 0, 64, 0, NULL, NULL) == 0
    assert L.cider_w4a8_gemm(NULL, NULL, NULL, NULL, 0, 16, 64, NULL, NULL) == 0
    assert L.cider_gemm_acc_i32(0, NULL, NULL, 0, 4, 64, 0, NULL, NULL) == 0
    assert L.cider_int8_mv(NULL, NULL, NULL, 0, 16, 64, 0, NULL, NULL) == 0
    assert L.cider_int8_mv(NULL, NULL, NULL, 2, 0, 64, 0, NULL, NULL) == 0
    assert L.cider_w8a8_gemm_token_group(NULL, NULL, NULL, NULL, 0, 16, 128, 64, NULL, NULL, 0, NULL) == 0
    assert L.cider_w8a8_gemm_token_group(NULL, NULL, NULL, NULL, 16, 0, 128, 128, NULL, NULL, 0, NULL) == 0


def test_quant_weight_rejects():
    assert L.cider_quant_weight(P, 4, 64, 6, 0, P, P, NULL) == INV        # bits
    assert L.cider_quant_weight(P, 4, 64, 4, 64, P, P, NULL) == INV       # int4 is per-channel
    assert L.cider_quant_weight(P, 4, 47, 4, 0, P, P, NULL) == INV        # int4 needs an even K
    assert L.cider_quant_weight(P, 4, 192, 8, 128, P, P, NULL) == INV     # K % gs
    assert L.cider_quant_weight(P, 4, 64, 8, 0, P, MIS, NULL) == INV


def test_gemm_rejects():
    g = L.cider_w8a8_gemm
    assert g(P, P, P, P, -1, 4, 64, 0, P, NULL) == INV
    assert g(P, P, P, P, 4, -1, 64, 0, P, NULL) == INV
    assert g(P, P, P, P, 4, 4, 0, 0, P, NULL) == INV
    assert g(P, P, P, P, 4, 4, 192, 128, P, NULL) == INV
    assert g(P, P, P, P, 4, 4, 128, 100, P, NULL) == INV
    assert g(P, P, P, P, 4, 4, 1 << 20, 0, P, NULL) == INV               # int32 range guard
    assert g(NULL, P, P, P, 4, 4, 64, 0, P, NULL) == INV
    assert g(P, P, P, P, 4, 4, 64, 0, NULL, NULL) == INV
    assert g(P, P, P, MIS, 4, 4, 64, 0, P, NULL) == INV
    h = L.cider_w4a8_gemm
    assert h(P, P, P, P, 4, 4, 47, P, NULL) == INV                      # int4 needs an even K
    assert h(P, P, MIS, P, 4, 4, 64, P, NULL) == INV
    a = L.cider_gemm_acc_i32
    assert a(2, P, P, 4, 4, 64, 0, P, NULL) == INV
    assert a(1, P, P, 4, 4, 64, 64, P, NULL) == INV
    assert a(0, P, P, 4, 4, 64, 0, NULL, NULL) == INV


def test_int8_mv_rejects():
    mv = L.cider_int8_mv
    assert mv(P, P, P, 5, 4, 64, 0, P, NULL) == INV                      # M above CIDER_MV_MAX_M
    assert mv(P, P, P, -1, 4, 64, 0, P, NULL) == INV
    assert mv(P, P, P, 1, 4, 40, 0, P, NULL) == INV                      # K % 16
    assert mv(P, P, P, 1, 4, 192, 128, P, NULL) == INV                   # K % gs
    assert mv(P, P, P, 1, 4, 128, 32, P, NULL) == INV                    # gs
    assert mv(NULL, P, P, 1, 4, 64, 0, P, NULL) == INV
    assert mv(P, P, NULL, 1, 4, 64, 0, P, NULL) == INV
    assert mv(MIS, P, P, 1, 4, 64, 0, P, NULL) == INV
    assert mv(P, P, P, 1, 4, 64, 0, MIS, NULL) == INV


def test_token_group_rejects():
    t = L.cider_w8a8_gemm_token_group
    assert t(P, P, P, P, 4, 4, 128, 0, P, NULL, 0, NULL) == INV                    # needs per-group weights
    assert t(P, P, P, P, 4, 4, 128, 32, P, NULL, 0, NULL) == INV
    assert t(P, P, P, P, 4, 4, 192, 128, P, NULL, 0, NULL) == INV                  # K % gs
    assert t(P, P, P, P, -1, 4, 128, 64, P, NULL, 0, NULL) == INV
    assert t(P, P, P, P, 4, 4, 133120 + 128, 64, P, NULL, 0, NULL) == INV          # int32 range guard
    assert t(NULL, P, P, P, 4, 4, 128, 64, P, NULL, 0, NULL) == INV
    assert t(P, NULL, P, P, 4, 4, 128, 64, P, NULL, 0, NULL) == INV
    assert t(P, P, P, P, 4, 4, 128, 64, NULL, NULL, 0, NULL) == INV
    assert t(P, MIS, P, P, 4, 4, 128, 64, P, NULL, 0, NULL) == INV


def test_split_rejects():
    sp = L.cider_w8a8_gemm_split
    n3 = (ctypes.c_int64 * 3)(32, 16, 48)
    y3 = (ctypes.c_void_p * 3)(1 << 20, 1 << 21, 1 << 22)
    cast = lambda a: ctypes.cast(a, ctypes.c_void_p)
    assert sp(P, P, P, P, 4, 64, 0, cast(n3), cast(y3), NULL) == INV        # no parts
    assert sp(P, P, P, P, 4, 64, 5, cast(n3), cast(y3), NULL) == INV        # above CIDER_SPLIT_MAX_PARTS
    bad = (ctypes.c_int64 * 3)(32, 8, 48)
    assert sp(P, P, P, P, 4, 64, 3, cast(bad), cast(y3), NULL) == INV       # width % 16
    zero = (ctypes.c_int64 * 3)(32, 0, 48)
    assert sp(P, P, P, P, 4, 64, 3, cast(zero), cast(y3), NULL) == INV
    assert sp(P, P, P, P, 4, 40, 3, cast(n3), cast(y3), NULL) == INV        # K % 16
    assert sp(P, P, P, P, 4, 64, 3, NULL, cast(y3), NULL) == INV
    ynull = (ctypes.c_void_p * 3)(1 << 20, None, 1 << 22)
    assert sp(P, P, P, P, 4, 64, 3, cast(n3), cast(ynull), NULL) == INV
    ymis = (ctypes.c_void_p * 3)(1 << 20, (1 << 21) + 8, 1 << 22)
    assert sp(P, P, P, P, 4, 64, 3, cast(n3), cast(ymis), NULL) == INV
    assert sp(NULL, P, P, P, 4, 64, 3, cast(n3), cast(y3), NULL) == INV
    assert sp(NULL, NULL, NULL, NULL, 0, 64, 3, cast(n3), cast(y3), NULL) == 0   # empty work


def test_linear_workspace_query_and_rejects():
    q = L.cider_linear_workspace_size
    assert q(1, 64, 2560, 8, 0) == 0 and q(2, 64, 32768, 8, 0) == 0 and q(2, 64, 2560, 4, 0) == 0   # one launch
    assert q(2, 64, 32768 + 256, 8, 0) == 2 * 33024 + 256                 # codes past the 64 KiB staging
    assert q(3, 64, 2560, 8, 0) == 3 * 2560 + 256                         # M = 3: separate quantization
    assert q(5, 64, 1024, 8, 0) == 5 * 1024 + 256
    assert q(5, 64, 1024, 8, 128) == 5 * 1024 + 256                       # 40 scale bytes
    assert q(300, 64, 1024, 8, 64) == 300 * 1024 + (4 * 300 * 16 + 255) // 256 * 256
    assert q(0, 64, 1024, 8, 0) == 0
    assert q(128, 2560, 10240, 8, 0) == 128 * 10240 + 512 + 8 * 128 * 2560 * 4   # + split-K slabs
    assert q(4, 64, 1024, 6, 0) == -1 and q(4, 64, 1024, 4, 64) == -1 and q(4, 64, 47, 4, 0) == -1
    # unaligned K: never the one-launch path, codes + scales through the workspace
    assert q(1, 64, 40, 8, 0) == 256 + 256 and q(2, 64, 34, 4, 0) == 256 + 256 and q(3, 64, 2568, 8, 0) == 7936 + 256
    assert q(-1, 64, 64, 8, 0) == -1
    lin = L.cider_linear
    assert lin(P, P, P, 4, 8, 1024, 6, 0, NULL, 0, P, NULL) == INV        # bits
    assert lin(P, P, P, 4, 8, 47, 4, 0, NULL, 0, P, NULL) == INV          # int4 needs an even K
    assert lin(P, P, P, 1, 8, 40, 8, 0, NULL, 0, P, NULL) == INV          # unaligned K needs the workspace
    assert lin(P, P, P, 5, 8, 1024, 8, 0, NULL, 0, P, NULL) == INV        # workspace needed
    assert lin(P, P, P, 5, 8, 1024, 8, 0, P, 100, P, NULL) == INV         # workspace too small
    assert lin(P, P, P, 5, 8, 1024, 8, 0, MIS, 1 << 20, P, NULL) == INV
    assert lin(NULL, P, P, 1, 8, 1024, 8, 0, NULL, 0, P, NULL) == INV
    assert lin(P, P, P, 1, 8, 1024, 8, 0, NULL, 0, MIS, NULL) == INV
    assert lin(NULL, NULL, NULL, 0, 8, 1024, 8, 0, NULL, 0, NULL, NULL) == 0  # empty work


def test_quant_weight_clip_rejects():
    c = L.cider_quant_weight_clip
    assert c(P, 0, 4, 64, 8, 0, 100.5, P, P, NULL) == INV               # percentile above 100
    assert c(P, 0, 4, 64, 8, 0, -0.1, P, P, NULL) == INV
    assert c(P, 0, 4, 64, 8, 0, float("nan"), P, P, NULL) == INV
    assert c(P, 2, 4, 64, 8, 0, 99.9, P, P, NULL) == INV                # dtype
    assert c(P, 0, 4, 64, 6, 0, 99.9, P, P, NULL) == INV                # bits
    assert c(P, 1, 4, 64, 4, 64, 99.9, P, P, NULL) == INV               # int4 is per-channel
    assert c(P, 0, 4, 48, 4, 0, 99.9, P, P, NULL) == INV                # int4 needs K % 32
    assert c(P, 0, 4, 192, 8, 128, 99.9, P, P, NULL) == INV             # K % gs
    assert c(P, 0, 4, 64, 8, 0, 99.9, P, MIS, NULL) == INV
    assert c(NULL, 0, 4, 64, 8, 0, 99.9, P, P, NULL) == INV
    assert c(NULL, 1, 0, 64, 8, 0, 99.9, NULL, NULL, NULL) == 0           # empty work


def test_dtype_entries_reject():
    assert L.cider_quant_act_dt(P, 2, 4, 64, 0, P, P, NULL) == INV      # dtype
    assert L.cider_quant_act_dt(P, -1, 4, 64, 0, P, P, NULL) == INV
    assert L.cider_quant_act_dt(P, 1, 4, 0, 0, P, P, NULL) == INV       # K >= 1
    assert L.cider_quant_act_dt(NULL, 1, 0, 64, 0, NULL, NULL, NULL) == 0
    assert L.cider_quant_weight_dt(P, 2, 4, 64, 8, 0, P, P, NULL) == INV
    assert L.cider_quant_weight_dt(P, 1, 4, 64, 4, 64, P, P, NULL) == INV
    assert L.cider_quant_weight_dt(NULL, 1, 0, 64, 8, 0, NULL, NULL, NULL) == 0
    assert L.cider_w8a8_gemm_dt(P, P, P, P, 4, 4, 64, 0, P, 2, NULL) == INV
    assert L.cider_w8a8_gemm_dt(P, P, P, P, 4, 4, 64, 0, MIS, 1, NULL) == INV
    assert L.cider_w8a8_gemm_dt(NULL, NULL, NULL, NULL, 0, 4, 64, 0, NULL, 1, NULL) == 0
    assert L.cider_w4a8_gemm_dt(P, P, P, P, 4, 4, 64, P, 7, NULL) == INV
    assert L.cider_w4a8_gemm_dt(P, P, P, P, 4, 4, 47, P, 1, NULL) == INV
    assert L.cider_w4a8_gemm_dt(NULL, NULL, NULL, NULL, 4, 0, 64, NULL, 1, NULL) == 0


def test_split_k_workspace_plan():
    g = L.cider_gemm_workspace_size
    assert g(128, 2560, 10240, 8, 0) == 8 * 128 * 2560 * 4        # 64x160 tiles, 8 K ranges
    assert g(1024, 2560, 10240, 8, 0) == 4 * 1024 * 2560 * 4      # 128x320 tiles, 4 K ranges
    assert g(128, 2560, 10240, 4, 0) == 8 * 128 * 2560 * 4        # W4A8: 128x128 tiles, 8 ranges
    assert g(4096, 10240, 2560, 8, 0) == 0                        # enough tiles: no split
    assert g(128, 10240, 2560, 8, 0) == 0                         # short K
    assert g(128, 2560, 10240, 8, 128) == 8 * 128 * 2560 * 4      # per-group: 64x160 tiles, 8 K ranges, fp32
    assert g(256, 2560, 10240, 8, 64) == 4 * 256 * 2560 * 4       # per-group: 64x64 tiles, 4 K ranges
    assert g(512, 2560, 10240, 8, 128) == 4 * 512 * 2560 * 4      # per-group: 128x128 tiles, 4 K ranges
    assert g(512, 2048, 4096, 8, 128) == 2 * 512 * 2048 * 4       # per-group, K < 8192: 64x64 tiles, 2 K ranges
    assert g(1024, 2560, 10240, 8, 128) == 3 * 1024 * 2560 * 4    # per-group: 128x128 tiles, 3 K ranges
    assert g(2048, 2560, 10240, 8, 128) == 2 * 2048 * 2560 * 4    # gs 128: 128x160 tiles, 2 K ranges
    assert g(2048, 2560, 10240, 8, 64) == 0                       # gs 64: 320 tiles of 128x128, no split
    assert g(4096, 2560, 10240, 8, 128) == 0                      # per-group with enough tiles
    assert g(16, 2560, 10240, 8, 0) == 0                          # skinny path
    assert g(0, 2560, 10240, 8, 0) == 0
    assert g(4, 4, 0, 8, 0) == -1 and g(4, 4, 64, 4, 64) == -1 and g(4, 4, 64, 6, 0) == -1
    assert g(4, 4, 47, 4, 0) == -1 and g(4, 4, 40, 8, 64) == -1
    assert g(4, 4, 40, 8, 0) == 0 and g(1024, 2560, 10248, 8, 0) == 0   # unaligned K never splits
    ex = L.cider_w8a8_gemm_ex
    assert ex(P, P, P, P, 128, 2560, 10240, 0, P, 0, P, 1024, NULL) == INV     # workspace too small
    assert ex(P, P, P, P, 128, 2560, 10240, 0, P, 0, MIS, 1 << 30, NULL) == INV
    assert ex(P, P, P, P, 128, 2560, 10240, 0, P, 3, NULL, 0, NULL) == INV     # dtype
    assert ex(NULL, NULL, NULL, NULL, 0, 2560, 10240, 0, NULL, 0, NULL, 0, NULL) == 0
    ex4 = L.cider_w4a8_gemm_ex
    assert ex4(P, P, P, P, 128, 2560, 10240, P, 0, P, 1024, NULL) == INV
    assert ex4(P, P, P, P, 128, 2560, 10240, P, 0, MIS, 1 << 30, NULL) == INV


def test_not_available_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert cider.cider_is_available() is False


def test_max_k_constant_keeps_int32_range():
    import re
    with open(cider.HEADER_PATH) as f:
        k = int(re.search(r"#define CIDER_MAX_K (\d+)", f.read()).group(1))
    assert 127 * 127 * k < 2 ** 31 and k % 128 == 0


def test_stack_layout_and_validation():
    import ctypes as ct
    offs = (ct.c_int64 * 9)()
    total = L.cider_stack_workspace_layout(64, 256, 256, 128, 512, offs)
    sizes = [64 * 512, 4 * 64, 2 * 64 * 256, 2 * 64 * 128, 2 * 64 * 128, 2 * 64 * 256, 2 * 64 * 512,
             2 * 64 * 512, 2 * 64 * 256]
    o = list(offs)
    assert o[0] == 0 and all(x % 256 == 0 for x in o)
    for i in range(8):
        assert o[i + 1] - o[i] >= sizes[i]
    assert total >= o[8] + sizes[8]
    assert L.cider_stack_workspace_layout(64, 250, 256, 128, 512, None) == 0
    layers = (cider.StackLayer * 1)()
    # null weight pointers are rejected before any HIP call
    assert L.cider_stack_forward(P, 64, 256, 256, 128, 512, 1, ct.cast(layers, ct.c_void_p), P, total, P,
                                 NULL) == INV
    assert L.cider_stack_forward(P, 64, 256, 256, 128, 512, 0, NULL, NULL, 0, NULL, NULL) == 0


def test_prepared_call_marshals_once_and_raises_on_error():
    ok = cider.prepared("cider_int8_mv", NULL, NULL, NULL, 0, 16, 64, 0, NULL, NULL)
    ok()
    ok()
    bad = cider.prepared("cider_int8_mv", P, P, P, 5, 4, 64, 0, P, NULL)
    with pytest.raises(Exception, match="cider_int8_mv"):
        bad()
