"""Plant plausible mistakes in copies of the CPU oracle and check that the pins
catch every one of them (CPU only; nothing here touches the GPU)."""
import types

import numpy as np
import pytest

from oracle import cider_oracle as O
from tests import oracle_pins as pins


def _impl(**over):
    base = {name: getattr(O, name) for name in (
        "quantize_rows", "pack_int4", "unpack_int4", "int_dot", "int_dot_groups",
        "dequant_per_channel", "dequant_per_group", "int8_mv", "dequant_token_group",
        "percentile_threshold", "quantize_rows_clip", "f64_to_bf16", "bf16_to_f32", "quantize_rows_bf16",
        "dequant_bf16", "dequant_token_group_bf16", "quantize_weight", "quantize_weight_clip",
        "quantize_weight_bf16", "quantize_weight_clip_bf16", "w8a8_linear", "w4a8_linear", "w8a8_linear_bf16",
        "w4a8_linear_bf16", "w8a8_linear_token_group", "w8a8_linear_token_group_bf16")}
    base.update(over)
    ns = types.SimpleNamespace(**base)
    return ns


def _quant_variant(rounding="even", divisor_bias=0, reciprocal=False, clamp=None):
    def q(X, group_size, qmax):
        R, K = X.shape
        G = O.num_groups(K, group_size)
        gs = K if group_size == 0 else group_size
        xg = X.astype(np.float32).reshape(R, G, gs)
        amax = np.abs(xg).max(axis=2)
        s = (amax / np.float32(qmax + divisor_bias)).astype(np.float32)
        zero = s == 0
        sd = np.where(zero, np.float32(1), s)[:, :, None]
        r = xg * (np.float32(1) / sd) if reciprocal else xg / sd
        t = np.floor(r + np.float32(0.5)) if rounding == "up" else np.rint(r)
        lo, hi = clamp if clamp else (-qmax, qmax)
        q = np.clip(t, lo, hi)
        q[zero] = 0
        return q.reshape(R, K).astype(np.int8), s
    return q


def _pack_swapped(q):
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 1::2] | (u[:, 0::2] << 4)).astype(np.uint8)


def _unpack_zp7(p):
    lo = (p & 0x0F).astype(np.int16) - 7
    hi = (p >> 4).astype(np.int16) - 7
    out = np.empty((p.shape[0], 2 * p.shape[1]), np.int16)
    out[:, 0::2], out[:, 1::2] = lo, hi
    return out.astype(np.int8)


def _dot_fp32(qa, qw):
    return (qa.astype(np.float32) @ qw.astype(np.float32).T).astype(np.int64)


def _dot_transposed(qa, qw):
    # right shapes only when M == N; otherwise the pins' shape checks fail
    k = min(qa.shape[0], qw.shape[0])
    out = O.int_dot(qa, qw)
    out[:k, :k] = out[:k, :k].T
    return out


def _dequant_no_sw(acc, s_a, s_w):
    return (acc.astype(np.float64) * s_a.astype(np.float64)[:, None]).astype(np.float16) * 0 + \
        (acc.astype(np.float64) * s_a.astype(np.float64)[:, None] * float(np.mean(s_w))).astype(np.float16)


def _dequant_sign(acc, s_a, s_w):
    y = O.dequant_per_channel(acc, s_a, s_w)
    y[..., -1] = -y[..., -1]
    return y


def _dequant_fp16_steps(acc, s_a, s_w):
    t = acc.astype(np.float16) * s_a.astype(np.float16)[:, None]
    return (t * s_w.astype(np.float16)[None, :]).astype(np.float16)


def _pg_drop_last_group(acc_g, s_a, s_w):
    return O.dequant_per_group(acc_g[:-1], s_a[:, :-1], s_w[:, :-1]) if acc_g.shape[0] > 1 \
        else O.dequant_per_group(acc_g, s_a, s_w)


def _pg_row_scale(acc_g, s_a, s_w):
    sa = np.repeat(s_a[:, :1], s_a.shape[1], axis=1)
    return O.dequant_per_group(acc_g, sa, s_w)


def _groups_off_by_one(qa, qw, group_size):
    out = O.int_dot_groups(qa, qw, group_size)
    if out.shape[0] > 1:
        out = np.roll(out, 1, axis=0)
    return out


def _mv_variant(kind):
    def mv(x, w_q, s_w, group_size=0):
        M, K = x.shape
        N = w_q.shape[0]
        G = O.num_groups(K, group_size)
        gs = K if group_size == 0 else group_size
        s = np.asarray(s_w, np.float32).reshape(N, G).astype(np.float64)
        if kind == "group_mod":            # scale index k % G instead of k // gs
            sk = s[:, np.arange(K) % G]
        else:
            sk = np.repeat(s, gs, axis=1)
        w = w_q.astype(np.float64) * sk
        xx = x.astype(np.float64)
        if kind == "no_scale":
            w = w_q.astype(np.float64)
        elif kind == "fp16_weights":       # dequantized weight rounded to fp16 first
            w = w.astype(np.float16).astype(np.float64)
        elif kind == "quantized_x":        # W8A8 semantics instead of fp16 activations
            qa, sa = O.quantize_rows(x, 0, 127)
            xx = qa.astype(np.float64) * sa.astype(np.float64)
        elif kind == "fp32_sum":
            return (x.astype(np.float32) @ w.astype(np.float32).T).astype(np.float16)
        return (xx @ w.T).astype(np.float16)
    return mv


def _tg_variant(kind):
    def f(acc_g, s_a, s_w):
        if kind == "no_act_scale":
            s_a = np.ones_like(s_a)
        elif kind == "first_group_scale":
            s_w = np.repeat(s_w[:, :1], s_w.shape[1], axis=1)
        elif kind == "reversed_groups":
            s_w = s_w[:, ::-1]
        return O.dequant_token_group(acc_g, s_a, s_w)
    return f


def _clip_variant(kind):
    """(threshold, quantizer) with one planted mistake in the percentile rule."""
    def threshold(mags, percentile):
        a = np.sort(np.asarray(mags, np.float64), axis=-1)
        if kind == "signed":
            a = np.sort(np.asarray(mags, np.float64) * np.where(np.arange(a.shape[-1]) % 2, -1, 1), axis=-1)
        n = a.shape[-1]
        h = float(n if kind == "n_not_n_minus_1" else n - 1) * (float(percentile) / 100.0)
        h = min(h, n - 1.0)
        i = int(np.floor(h))
        j = min(i + 1, n - 1)
        g = h - i
        if kind == "lower":
            t = a[..., i]
        elif kind == "higher":
            t = a[..., j]
        elif kind == "max":
            t = a[..., -1]
        else:
            t = a[..., i] + g * (a[..., j] - a[..., i])
        return t.astype(np.float32)

    def quant(X, group_size, qmax, percentile):
        R, K = X.shape
        G = O.num_groups(K, group_size)
        gs = K if group_size == 0 else group_size
        xg = X.astype(np.float32).reshape(R, G, gs)
        s = (threshold(np.abs(xg), percentile) / np.float32(qmax)).astype(np.float32)
        zero = s == 0
        r = xg / np.where(zero, np.float32(1), s)[:, :, None]
        q = np.rint(r) if kind == "no_saturation" else np.clip(np.rint(r), -qmax, qmax)
        q[zero] = 0
        return q.reshape(R, K).astype(np.int8 if kind != "no_saturation" else np.int64), s
    return threshold, quant


def _clip_impl(kind):
    t, q = _clip_variant(kind)
    return _impl(percentile_threshold=t, quantize_rows_clip=q)


def _bf16_variant(kind):
    """(rounding, dequant, quantizer) with one planted bf16 mistake."""
    def rnd(v):
        v = np.asarray(v, np.float64)
        if kind == "truncate":
            return (v.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
        if kind == "via_fp32":
            f = v.astype(np.float32).view(np.uint32)
            r = (f + np.uint32(0x7FFF) + ((f >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
            return r.astype(np.uint16)
        return O.f64_to_bf16(v)

    def deq(acc_g, s_a, s_w):
        if acc_g.ndim == 2:
            return rnd(acc_g.astype(np.float64) * s_a.astype(np.float64)[:, None] * s_w.astype(np.float64)[None, :])
        y = np.zeros(acc_g.shape[1:], np.float64)
        for g in range(acc_g.shape[0]):
            y += acc_g[g].astype(np.float64) * s_a[:, g].astype(np.float64)[:, None] * s_w[:, g].astype(np.float64)[None, :]
        return rnd(y)

    def quant(Xbits, group_size, qmax):
        if kind == "as_fp16":
            return O.quantize_rows(np.asarray(Xbits, np.uint16).view(np.float16), group_size, qmax)
        return O.quantize_rows_bf16(Xbits, group_size, qmax)
    return _impl(f64_to_bf16=rnd, dequant_bf16=deq, quantize_rows_bf16=quant)


def _tok_bf16_no_act_scale(acc_g, s_a, s_w):
    return O.dequant_token_group_bf16(acc_g, np.ones_like(s_a), s_w)


def _dequant_fp64_two_roundings(acc, s_a, s_w):
    # the product rounded to fp64 and then to fp16: wrong at constructed midpoints
    t = acc.astype(np.float64) * s_a.astype(np.float64)[:, None]
    return (t * s_w.astype(np.float64)[None, :]).astype(np.float16)


def _clip_int4_unpacked(w, bits=8, group_size=0, percentile=99.9):
    if bits == 4:   # the int4 codes returned without packing them
        q, s = O.quantize_rows_clip(w, 0, 7, percentile)
        return q, s[:, 0]
    return O.quantize_weight_clip(w, bits, group_size, percentile)


def _weight_bf16_as_fp16(w_bits, bits=8, group_size=0):
    return O.quantize_weight(np.asarray(w_bits, np.uint16).view(np.float16), bits, group_size)


def _clip_bf16_min_max(w_bits, bits=8, group_size=0, percentile=99.9):
    return O.quantize_weight_bf16(w_bits, bits, group_size)


def _linear_bf16_act_per_token(x_bits, w_q, s_w, group_size=0):
    # per-group weights, but the activations quantized per token
    if group_size == 0:
        return O.w8a8_linear_bf16(x_bits, w_q, s_w, 0)
    q_a, s2 = O.quantize_rows_bf16(x_bits, 0, 127)
    sa = np.repeat(s2, s_w.shape[1], axis=1)
    return O.dequant_bf16(O.int_dot_groups(q_a, w_q, group_size), sa, s_w), q_a, sa


def _w4a8_bf16_swapped_nibbles(x_bits, w_packed, s_w):
    p = np.asarray(w_packed, np.uint8)
    return O.w4a8_linear_bf16(x_bits, ((p >> 4) | (p << 4)).astype(np.uint8), s_w)


def _token_group_act_per_group(x, w_q, s_w, group_size):
    q_a, s_a = O.quantize_rows(x, group_size, 127)   # per-group activation codes
    y = O.dequant_per_group(O.int_dot_groups(q_a, w_q, group_size), s_a, s_w)
    return y, q_a, s_a[:, 0]


def _token_group_bf16_fp16_output(x_bits, w_q, s_w, group_size):
    y, q_a, s_a = O.w8a8_linear_token_group_bf16(x_bits, w_q, s_w, group_size)
    f = O.bf16_to_f32(y)
    return f.astype(np.float16).view(np.uint16), q_a, s_a


MUTANTS = {
    "round_half_up": _impl(quantize_rows=_quant_variant(rounding="up")),
    "scale_over_128": _impl(quantize_rows=_quant_variant(divisor_bias=1)),
    "reciprocal_multiply": _impl(quantize_rows=_quant_variant(reciprocal=True)),
    "clamp_to_126": _impl(quantize_rows=_quant_variant(clamp=(-126, 126))),
    "int4_nibbles_swapped": _impl(pack_int4=_pack_swapped),
    "int4_zero_point_7": _impl(unpack_int4=_unpack_zp7),
    "fp32_accumulation": _impl(int_dot=_dot_fp32),
    "transposed_output": _impl(int_dot=_dot_transposed),
    "dropped_weight_scale": _impl(dequant_per_channel=_dequant_no_sw),
    "sign_flip_last_column": _impl(dequant_per_channel=_dequant_sign),
    "fp16_dequant_steps": _impl(dequant_per_channel=_dequant_fp16_steps),
    "per_group_drops_a_group": _impl(dequant_per_group=_pg_drop_last_group),
    "per_group_row_scale": _impl(dequant_per_group=_pg_row_scale),
    "per_group_misaligned": _impl(int_dot_groups=_groups_off_by_one),
    "mv_without_weight_scale": _impl(int8_mv=_mv_variant("no_scale")),
    "mv_group_index_modulo": _impl(int8_mv=_mv_variant("group_mod")),
    "mv_fp16_dequantized_weight": _impl(int8_mv=_mv_variant("fp16_weights")),
    "mv_quantizes_activations": _impl(int8_mv=_mv_variant("quantized_x")),
    "mv_fp32_sum": _impl(int8_mv=_mv_variant("fp32_sum")),
    "token_group_without_act_scale": _impl(dequant_token_group=_tg_variant("no_act_scale")),
    "token_group_first_weight_scale": _impl(dequant_token_group=_tg_variant("first_group_scale")),
    "token_group_reversed_scales": _impl(dequant_token_group=_tg_variant("reversed_groups")),
    "clip_position_n": _clip_impl("n_not_n_minus_1"),
    "clip_lower_order_statistic": _clip_impl("lower"),
    "clip_higher_order_statistic": _clip_impl("higher"),
    "clip_ignores_percentile": _clip_impl("max"),
    "clip_signed_values": _clip_impl("signed"),
    "clip_no_saturation": _clip_impl("no_saturation"),
    "bf16_truncation": _bf16_variant("truncate"),
    "bf16_double_rounding_via_fp32": _bf16_variant("via_fp32"),
    "bf16_rows_read_as_fp16": _bf16_variant("as_fp16"),
    "token_group_bf16_no_act_scale": _impl(dequant_token_group_bf16=_tok_bf16_no_act_scale),
    "dequant_fp64_double_rounding": _impl(dequant_per_channel=_dequant_fp64_two_roundings),
    "clip_int4_not_packed": _impl(quantize_weight_clip=_clip_int4_unpacked),
    "weight_bf16_read_as_fp16": _impl(quantize_weight_bf16=_weight_bf16_as_fp16),
    "clip_bf16_ignores_percentile": _impl(quantize_weight_clip_bf16=_clip_bf16_min_max),
    "linear_bf16_per_token_activations": _impl(w8a8_linear_bf16=_linear_bf16_act_per_token),
    "w4a8_bf16_swapped_nibbles": _impl(w4a8_linear_bf16=_w4a8_bf16_swapped_nibbles),
    "token_group_quantizes_per_group": _impl(w8a8_linear_token_group=_token_group_act_per_group),
    "token_group_bf16_fp16_output": _impl(w8a8_linear_token_group_bf16=_token_group_bf16_fp16_output),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = MUTANTS[name]
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"
