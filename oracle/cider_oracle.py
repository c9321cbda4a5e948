"""Plain, slow CPU oracle of Cider's online-quantized linear layer (W8A8 / W4A8).

TEST INFRASTRUCTURE. Only the test suite, the package's smoke check and the
CPU-baseline leg of the benchmark may import or run this module. The HIP
library never calls it, shares no code with it, and must not fall back to it.

What it computes, and where the pages say so (all citations are to the
top-level Cider README, a community translation of the upstream README):

* Section "模式" (Modes) table: W8A8 = symmetric INT8 weights with INT8
  per-token activations; W4A8 = INT4 weights packed in uint8 with INT8
  per-token activations.
* Section "W8A8 量化粒度" (W8A8 quantization granularity) table: per-channel
  (one scale per output channel) or per-group (one scale per 128 or per 64
  elements).
* Section "架构 / Metal Kernel 流水线" (kernel pipeline): prefill first turns
  fp16 activations into int8 plus one scale per token, then runs an
  INT8 x INT8 -> INT32 matmul whose store stage dequantizes to fp16; for
  W4A8 the int4 weights are unpacked to int8 while the fragments are loaded.
* Section "量化" (Quantization) table: weights symmetric INT8 (per-channel or
  per-group gs=64/128) or symmetric INT4 with zero point 8 per column;
  activations symmetric INT8 per token; INT32 accumulation; the output is
  the int32 accumulator times the activation scale times the weight scale,
  per element, in fp16.
* Section "说明" (Notes): scales come from the min-max rule by default; a
  percentile rule (clip_percentile=99.9) is offered as well.
* Section "架构 / Metal Kernel 流水线", Decode (M = 1): int8_mv multiplies
  fp16 activations by int8 weights dequantized on the fly, without
  quantizing the activations (per-channel and per-group MV kernels in the
  file list).

Readings taken where the pages are silent (each is also listed in the design
notes of the repository):

* scale = max|v| / qmax over the row (or group), qmax = 127 for int8 and 7
  for int4, computed in fp32 with one correctly rounded division; stored as
  fp32.
* code = clamp(round_half_even(v / scale), -qmax, qmax), with v / scale one
  correctly rounded fp32 division. The fp32 precision of this decision is
  the kernel's (the pages fix none); -128 is never produced.
* a row or group whose max|v| is 0 gets scale 0 and all codes 0.
* per-group (gs = 64 or 128) groups run along K and apply to the activation
  and the weight alike: y = sum_g acc_g * s_a[m,g] * s_w[n,g].
* int4: codes in [-7, 7] stored as nibble u = code + 8; two codes per byte,
  the even K index in the low nibble; weight rows are [N, K/2] bytes.
* dequant: the exact product acc * s_a * s_w (summed over groups for
  per-group) rounded to fp16 (round to nearest even). Per-channel, this is
  the plain definition rounded exactly once: the fp64 route is used where it
  provably gives that result (|acc| < 2^29, so acc * s_a is exact in fp64,
  and the fp64 product is not a midpoint of the output format, so its second
  rounding cannot land on the wrong side), and every other element is
  computed with exact rationals. Per-group sums are evaluated in fp64: each
  term acc_g * s_a * s_w is rounded once to fp64 (|acc_g| < 2^29 for the
  group sizes accepted) and the sum over G groups carries at most about
  G * 2^-53 * sum_g |term_g| of error before the final fp16 rounding; the
  GPU's fp32 sums are held to a much wider bound.

* per-token activations x per-group weights (the quantization table's
  per-token activations with per-group weights): y = sum_g acc_g * s_a[m] *
  s_w[n,g], evaluated in fp64 as the per-group sum is, then rounded to fp16.
* percentile-clipped weight scales (the notes name a "99th percentile"
  method with clip_percentile=99.9; the parameter's value is taken): the
  group's clip threshold t is the percentile of its magnitudes by linear
  interpolation between order statistics (numpy's default definition),
  evaluated as written in fp64 and rounded to fp32; s = t / qmax and the
  codes follow the min-max rule's code step, so magnitudes above t saturate.
* bf16 I/O (the roadmap's automatic float16 / bfloat16 handling): bf16
  activations and weights quantize by the same rule (their fp32 images are
  exact); the output is the same exact dequant value rounded once to bf16.
* decode MV: y = sum_k x[m,k] * (w_q[n,k] * s_w[n,g(k)]), the exact value
  rounded once to fp16 (evaluated in fp64: each product is exact, the sum's
  relative error is about K * 2^-53).

Integer accumulation is done as an fp64 matmul of int8-valued arrays. Every
product and partial sum is an integer of magnitude at most 127*127*K, which
is below 2**53 for every K this module accepts, so each fp64 operation
(whatever the BLAS blocking order or FMA use) is exact.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "QMAX_INT8", "QMAX_INT4", "quantize_rows", "quantize_act", "quantize_weight",
    "pack_int4", "unpack_int4", "int_dot", "int_dot_groups", "dequant_per_channel",
    "dequant_per_group", "w8a8_linear", "w4a8_linear", "num_groups", "int8_mv",
    "dequant_token_group", "w8a8_linear_token_group", "percentile_threshold", "quantize_rows_clip",
    "quantize_weight_clip", "bf16_to_f32", "f64_to_bf16", "quantize_rows_bf16", "quantize_weight_bf16",
    "quantize_weight_clip_bf16", "dequant_bf16", "w8a8_linear_bf16", "w4a8_linear_bf16",
    "dequant_token_group_bf16", "w8a8_linear_token_group_bf16",
]

QMAX_INT8 = 127
QMAX_INT4 = 7
_EXACT_K_LIMIT = (2 ** 53) // (127 * 127)


def num_groups(K: int, group_size: int) -> int:
    """G = 1 for per-row scales (group_size 0), else K / group_size."""
    if group_size == 0:
        return 1
    if K % group_size:
        raise ValueError(f"K={K} is not a multiple of group_size={group_size}")
    return K // group_size


def quantize_rows(X: np.ndarray, group_size: int, qmax: int):
    """Symmetric min-max quantization of every row (or K-group of a row).

    X: fp16 [R, K]. group_size 0 = one scale per row; otherwise one scale per
    run of group_size consecutive K elements. Returns (q int8 [R, K],
    s fp32 [R, G]).
    """
    X = np.asarray(X)
    if X.dtype != np.float16 or X.ndim != 2:
        raise TypeError("X must be a 2-D float16 array")
    R, K = X.shape
    G = num_groups(K, group_size)
    gs = K if group_size == 0 else group_size
    return _quantize_values(X.astype(np.float32), group_size, qmax)   # fp16 -> fp32 is exact


def _quantize_values(Xf: np.ndarray, group_size: int, qmax: int):
    """The min-max steps on fp32 values (exact images of fp16 or bf16 inputs)."""
    R, K = Xf.shape
    G = num_groups(K, group_size)
    gs = K if group_size == 0 else group_size
    xg = Xf.reshape(R, G, gs)
    amax = np.abs(xg).max(axis=2) if K else np.zeros((R, G), np.float32)
    s = (amax / np.float32(qmax)).astype(np.float32)      # one rounded fp32 division
    zero = s == 0
    r = xg / np.where(zero, np.float32(1), s)[:, :, None]  # one rounded fp32 division
    q = np.clip(np.rint(r), -qmax, qmax)                   # rint: ties to even
    q[zero] = 0
    return q.reshape(R, K).astype(np.int8), s


def quantize_act(x: np.ndarray, group_size: int = 0):
    """Per-token (group_size 0) or per-group int8 activation quantization.

    Returns (q int8 [M, K], s fp32 [M] for per-token, [M, K/gs] per-group)."""
    q, s = quantize_rows(x, group_size, QMAX_INT8)
    return q, (s[:, 0] if group_size == 0 else s)


def quantize_weight(w: np.ndarray, bits: int = 8, group_size: int = 0):
    """Weight quantization, offline (the README's low-level API section shows
    the weight quantizers running in numpy before any kernel call).

    bits 8: int8 [N, K] codes with fp32 scales [N] (group_size 0) or [N, K/gs].
    bits 4: packed uint8 [N, K/2] (low nibble = even k) with fp32 scales [N].
    """
    if bits == 8:
        q, s = quantize_rows(w, group_size, QMAX_INT8)
        return q, (s[:, 0] if group_size == 0 else s)
    if bits == 4:
        if group_size != 0:
            raise ValueError("int4 weights are per output channel only")
        q, s = quantize_rows(w, 0, QMAX_INT4)
        return pack_int4(q), s[:, 0]
    raise ValueError("bits must be 8 or 4")


def percentile_threshold(mags: np.ndarray, percentile: float) -> np.ndarray:
    """Clip threshold of each group for percentile-clipped scales (the README's
    notes section: scales by min-max by default, or by a percentile of the
    magnitudes, clip_percentile=99.9).

    mags: [..., n] magnitudes (exact fp16 values). The percentile is taken by
    linear interpolation between order statistics: with a the magnitudes in
    ascending order, position h = (n - 1) * (percentile / 100), i = floor(h),
    j = min(i + 1, n - 1): t = a[i] + (h - i) * (a[j] - a[i]). Every step is
    one rounded fp64 operation in that order (no fused multiply-add); t is
    then rounded to fp32. Returns fp32 [...].
    """
    a = np.sort(np.asarray(mags, np.float64), axis=-1)
    n = a.shape[-1]
    h = float(n - 1) * (float(percentile) / 100.0)
    i = int(np.floor(h))
    j = min(i + 1, n - 1)
    g = h - i
    lo, hi = a[..., i], a[..., j]
    t = lo + g * (hi - lo)            # numpy rounds the product, then the sum
    return t.astype(np.float32)


def quantize_rows_clip(X: np.ndarray, group_size: int, qmax: int, percentile: float):
    """As quantize_rows, with each group's scale s = t / qmax (one rounded fp32
    division) for t = percentile_threshold of the group's magnitudes instead
    of max|v|. Codes follow the same rule, clamp(rint(v / s), -qmax, qmax),
    so magnitudes above t saturate at +-qmax; s == 0 gives codes 0."""
    X = np.asarray(X)
    if X.dtype != np.float16 or X.ndim != 2:
        raise TypeError("X must be a 2-D float16 array")
    if not 0.0 <= percentile <= 100.0:
        raise ValueError("percentile must lie in [0, 100]")
    return _quantize_clip_values(X.astype(np.float32), group_size, qmax, percentile)


def _quantize_clip_values(Xf: np.ndarray, group_size: int, qmax: int, percentile: float):
    """The percentile-clipped steps on fp32 values (exact images of the inputs)."""
    R, K = Xf.shape
    G = num_groups(K, group_size)
    gs = K if group_size == 0 else group_size
    xg = Xf.reshape(R, G, gs)
    t = percentile_threshold(np.abs(xg), percentile)
    s = (t / np.float32(qmax)).astype(np.float32)
    zero = s == 0
    r = xg / np.where(zero, np.float32(1), s)[:, :, None]
    q = np.clip(np.rint(r), -qmax, qmax)
    q[zero] = 0
    return q.reshape(R, K).astype(np.int8), s


def quantize_weight_clip(w: np.ndarray, bits: int = 8, group_size: int = 0, percentile: float = 99.9):
    """quantize_weight with percentile-clipped scales (same outputs and layouts)."""
    if bits == 8:
        q, s = quantize_rows_clip(w, group_size, QMAX_INT8, percentile)
        return q, (s[:, 0] if group_size == 0 else s)
    if bits == 4:
        if group_size != 0:
            raise ValueError("int4 weights are per output channel only")
        q, s = quantize_rows_clip(w, 0, QMAX_INT4, percentile)
        return pack_int4(q), s[:, 0]
    raise ValueError("bits must be 8 or 4")


def pack_int4(q: np.ndarray) -> np.ndarray:
    """Codes in [-7, 7], [N, K] with K even -> uint8 [N, K/2].

    Byte j of a row holds code 2j (plus 8) in its low nibble and code 2j+1
    (plus 8) in its high nibble."""
    q = np.asarray(q)
    if q.shape[1] % 2:
        raise ValueError("K must be even to pack int4")
    if q.size and (q.min() < -QMAX_INT4 or q.max() > QMAX_INT4):
        raise ValueError("int4 codes must lie in [-7, 7]")
    u = (q.astype(np.int16) + 8).astype(np.uint8)
    return (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(p: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4: uint8 [N, K/2] -> int8 codes [N, K]."""
    p = np.asarray(p, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16) - 8
    hi = (p >> 4).astype(np.int16) - 8
    out = np.empty((p.shape[0], 2 * p.shape[1]), np.int16)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out.astype(np.int8)


def int_dot(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k qa[m, k] * qw[n, k], exact, as int64 [M, N]."""
    K = qa.shape[1]
    if qw.shape[1] != K:
        raise ValueError("K mismatch")
    if K > _EXACT_K_LIMIT:
        raise ValueError("K too large for an exact fp64 integer dot product")
    return (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def int_dot_groups(qa: np.ndarray, qw: np.ndarray, group_size: int) -> np.ndarray:
    """Per-group exact dot products: acc[g, m, n] over k in group g, int64."""
    K = qa.shape[1]
    G = num_groups(K, group_size)
    gs = K if group_size == 0 else group_size
    return np.stack([int_dot(qa[:, g * gs:(g + 1) * gs], qw[:, g * gs:(g + 1) * gs])
                     for g in range(G)])


# Output formats of the dequant: (significand bits including the hidden one,
# smallest normal exponent, largest exponent).
_F16 = (11, -14, 15)
_BF16 = (8, -126, 127)


def _round_rational(v: Fraction, fmt) -> float:
    """The exact rational v rounded once to the binary format fmt (nearest,
    ties to the even significand, gradual underflow, +-inf once the rounded
    magnitude reaches 2^(emax+1)), as a Python float."""
    p, emin, emax = fmt
    if v == 0:
        return 0.0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # 2^(e-1) < a < 2^(e+1)
    if a < Fraction(2) ** e:
        e -= 1
    step = Fraction(2) ** (max(e, emin) - (p - 1))              # spacing of the format at a
    n, rem = divmod(a, step)
    if 2 * rem > step or (2 * rem == step and n % 2 == 1):
        n += 1
    r = n * step
    out = math.inf if r >= Fraction(2) ** (emax + 1) else float(r)
    return -out if v < 0 else out


def _is_midpoint(p: np.ndarray, fmt) -> np.ndarray:
    """True where the fp64 value p lies exactly halfway between two
    neighbours of the format (where rounding p again could differ from
    rounding the exact value it came from)."""
    bits, emin, _ = fmt
    a = np.abs(p)
    _, e = np.frexp(a)                                   # 2^(e-1) <= a < 2^e
    q = np.maximum(e - 1, emin) - (bits - 1)              # exponent of the spacing
    n = np.ldexp(a, -q)                                   # exact: a power-of-two scaling
    return (a != 0) & (n - np.floor(n) == 0.5)


def _product_rounded(acc: np.ndarray, s_a: np.ndarray, s_w: np.ndarray, fmt, to_fmt):
    """acc[m, n] * s_a[m] * s_w[n] rounded once to fmt: fp64 where that is
    provably the same, exact rationals elsewhere. Returns to_fmt(values)."""
    acc = np.asarray(acc)
    sa64 = s_a.astype(np.float64)[:, None]
    sw64 = s_w.astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        t = acc.astype(np.float64) * sa64                  # exact while |acc| < 2^29
        v = t * sw64
    redo = (np.abs(acc) >= 2 ** 29) | _is_midpoint(v, fmt) | ~np.isfinite(v)
    for m, n in zip(*np.nonzero(redo)):
        exact = Fraction(int(acc[m, n])) * Fraction(float(s_a[m])) * Fraction(float(s_w[n]))
        v[m, n] = _round_rational(exact, fmt)
    return to_fmt(v)


def dequant_per_channel(acc: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """y[m, n] = fp16(acc[m, n] * s_a[m] * s_w[n]): the exact product rounded once
    to fp16. (Where the fp64 route is used the value handed to the fp16 cast
    is either the exact product or lies strictly on the same side of every
    fp16 rounding boundary as it, so the cast gives the single rounding.)"""
    with np.errstate(over="ignore"):
        return _product_rounded(acc, s_a, s_w, _F16, lambda v: v.astype(np.float16))


def dequant_per_group(acc_g: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """y[m, n] = fp16(sum_g acc_g[g, m, n] * s_a[m, g] * s_w[n, g]), the sum in fp64
    (each term rounded once to fp64; see the module notes for its error)."""
    G = acc_g.shape[0]
    y = np.zeros(acc_g.shape[1:], np.float64)
    for g in range(G):
        t = acc_g[g].astype(np.float64) * s_a[:, g].astype(np.float64)[:, None]
        y += t * s_w[:, g].astype(np.float64)[None, :]
    return y.astype(np.float16)


def w8a8_linear(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int = 0):
    """The full online W8A8 linear: quantize x, integer matmul, dequant to fp16.

    Returns (y fp16 [M, N], q_a int8 [M, K], s_a fp32)."""
    q_a, s_a = quantize_act(x, group_size)
    if group_size == 0:
        y = dequant_per_channel(int_dot(q_a, w_q), s_a, s_w)
    else:
        y = dequant_per_group(int_dot_groups(q_a, w_q, group_size), s_a, s_w)
    return y, q_a, s_a


# ------------------------------------------------------------------ bf16 I/O
# The README's roadmap lists automatic float16 / bfloat16 handling: a bf16
# model feeds bf16 activations (and weights) and gets bf16 outputs. numpy has
# no bfloat16, so bf16 arrays are carried as uint16 bit patterns (the top half
# of the fp32 pattern). The quantization rule is unchanged (bf16 -> fp32 is
# exact); the dequantized output is rounded once to bf16 instead of fp16.

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns -> the fp32 values they denote (exact)."""
    b = np.asarray(bits, np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f64_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values once to bfloat16 (nearest, ties to even; 8 significand
    bits, exponents of fp32, gradual underflow below 2^-126, +-inf from
    2^128 up). Returns uint16 bit patterns."""
    v = np.asarray(v, np.float64)
    a = np.abs(v)
    _, e = np.frexp(a)                                  # 2^(e-1) <= a < 2^e
    q = np.maximum(e - 1, -126) - 7                     # exponent of the bf16 spacing
    val = np.ldexp(np.rint(np.ldexp(a, -q)), q)          # exact scalings; one rounding
    val = np.where(val >= 2.0 ** 128, np.inf, val)
    bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.signbit(v), bits | np.uint16(0x8000), bits).astype(np.uint16)


def quantize_rows_bf16(Xbits: np.ndarray, group_size: int, qmax: int):
    """quantize_rows for bf16 rows (uint16 patterns [R, K])."""
    Xbits = np.asarray(Xbits)
    if Xbits.dtype != np.uint16 or Xbits.ndim != 2:
        raise TypeError("Xbits must be a 2-D uint16 array of bf16 patterns")
    return _quantize_values(bf16_to_f32(Xbits), group_size, qmax)


def quantize_weight_bf16(w_bits: np.ndarray, bits: int = 8, group_size: int = 0):
    """quantize_weight for bf16 weights (same outputs and layouts)."""
    if bits == 8:
        q, s = quantize_rows_bf16(w_bits, group_size, QMAX_INT8)
        return q, (s[:, 0] if group_size == 0 else s)
    if bits == 4:
        if group_size != 0:
            raise ValueError("int4 weights are per output channel only")
        q, s = quantize_rows_bf16(w_bits, 0, QMAX_INT4)
        return pack_int4(q), s[:, 0]
    raise ValueError("bits must be 8 or 4")


def quantize_weight_clip_bf16(w_bits: np.ndarray, bits: int = 8, group_size: int = 0, percentile: float = 99.9):
    """quantize_weight_clip for bf16 weights (uint16 patterns)."""
    if not 0.0 <= percentile <= 100.0:
        raise ValueError("percentile must lie in [0, 100]")
    qmax = QMAX_INT8 if bits == 8 else QMAX_INT4
    if bits == 4 and group_size != 0:
        raise ValueError("int4 weights are per output channel only")
    q, s = _quantize_clip_values(bf16_to_f32(np.asarray(w_bits, np.uint16)), group_size, qmax, percentile)
    if bits == 4:
        return pack_int4(q), s[:, 0]
    return q, (s[:, 0] if group_size == 0 else s)


def dequant_bf16(acc_g: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """Per-channel (acc [M, N], s_a [M], s_w [N]) or per-group (acc_g [G, M, N],
    s_a [M, G], s_w [N, G]) dequant, the exact fp64 value rounded once to
    bf16 (uint16 patterns [M, N])."""
    if acc_g.ndim == 2:
        return _product_rounded(acc_g, s_a, s_w, _BF16, f64_to_bf16)
    y = np.zeros(acc_g.shape[1:], np.float64)
    for g in range(acc_g.shape[0]):
        t = acc_g[g].astype(np.float64) * s_a[:, g].astype(np.float64)[:, None]
        y += t * s_w[:, g].astype(np.float64)[None, :]
    return f64_to_bf16(y)


def w8a8_linear_bf16(x_bits: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int = 0):
    """w8a8_linear with bf16 activations in and bf16 output (uint16 patterns).
    Returns (y [M, N], q_a, s_a)."""
    q_a, s2 = quantize_rows_bf16(x_bits, group_size, QMAX_INT8)
    if group_size == 0:
        y = dequant_bf16(int_dot(q_a, w_q), s2[:, 0], s_w)
        return y, q_a, s2[:, 0]
    return dequant_bf16(int_dot_groups(q_a, w_q, group_size), s2, s_w), q_a, s2


def w4a8_linear_bf16(x_bits: np.ndarray, w_packed: np.ndarray, s_w: np.ndarray):
    """w4a8_linear with bf16 activations in and bf16 output."""
    q_a, s2 = quantize_rows_bf16(x_bits, 0, QMAX_INT8)
    return dequant_bf16(int_dot(q_a, unpack_int4(w_packed)), s2[:, 0], s_w), q_a, s2[:, 0]


def w4a8_linear(x: np.ndarray, w_packed: np.ndarray, s_w: np.ndarray):
    """W4A8: per-token int8 activations times unpacked int4 weights, per-channel."""
    q_a, s_a = quantize_act(x, 0)
    y = dequant_per_channel(int_dot(q_a, unpack_int4(w_packed)), s_a, s_w)
    return y, q_a, s_a


def int8_mv(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int = 0) -> np.ndarray:
    """Decode matrix-vector product (README section "架构 / Metal Kernel 流水线",
    Decode (M = 1): int8_mv multiplies fp16 activations by int8 weights that are
    dequantized on the fly, with no activation quantization; the README's file
    list names a per-channel and a per-group MV kernel).

    y[m, n] = fp16( sum_k x[m, k] * (w_q[n, k] * s_w[n, g(k)]) ), g(k) = k // group_size
    (g = 0 for per-channel, group_size 0). x is fp16 [M, K], w_q int8 [N, K],
    s_w fp32 [N] or [N, K / group_size].

    The dequantized weight w_q * s_w is exact in fp64 (8 + 24 significant bits)
    and so is its product with an fp16 activation; the sum over k is an fp64
    matmul (relative error about K * 2^-53, far below the one fp16 rounding that
    follows). This is the plain definition, rounded once."""
    M, K = x.shape
    N = w_q.shape[0]
    G = num_groups(K, group_size)
    gs = K if group_size == 0 else group_size
    s = np.asarray(s_w, np.float32).reshape(N, G).astype(np.float64)
    w_deq = w_q.astype(np.float64) * np.repeat(s, gs, axis=1)
    with np.errstate(over="ignore"):
        return (x.astype(np.float64) @ w_deq.T).astype(np.float16)


def dequant_token_group(acc_g: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """Per-token activation scale times per-group weight scales (the README's
    quantization table: activations symmetric INT8 per token in every mode,
    weights per-channel or per-group): y[m, n] = fp16( sum_g acc_g[g, m, n] *
    s_a[m] * s_w[n, g] ), evaluated in fp64 (acc_g * s_a exact, each term then
    rounded once to fp64, the sum carrying at most about G * 2^-53 of the
    terms' magnitude), then rounded to fp16."""
    G = acc_g.shape[0]
    sa = s_a.reshape(-1).astype(np.float64)[:, None]
    y = np.zeros(acc_g.shape[1:], np.float64)
    for g in range(G):
        y += (acc_g[g].astype(np.float64) * sa) * s_w[:, g].astype(np.float64)[None, :]
    with np.errstate(over="ignore"):
        return y.astype(np.float16)


def dequant_token_group_bf16(acc_g: np.ndarray, s_a: np.ndarray, s_w: np.ndarray) -> np.ndarray:
    """dequant_token_group with a bfloat16 output: the same fp64 value
    sum_g acc_g[g, m, n] * s_a[m] * s_w[n, g], rounded once to bf16 (uint16
    patterns [M, N])."""
    G = acc_g.shape[0]
    sa = s_a.reshape(-1).astype(np.float64)[:, None]
    y = np.zeros(acc_g.shape[1:], np.float64)
    for g in range(G):
        y += (acc_g[g].astype(np.float64) * sa) * s_w[:, g].astype(np.float64)[None, :]
    return f64_to_bf16(y)


def w8a8_linear_token_group_bf16(x_bits: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int):
    """w8a8_linear_token_group with bf16 activations in (uint16 patterns) and
    a bf16 output. Returns (y, q_a, s_a)."""
    q_a, s2 = quantize_rows_bf16(x_bits, 0, QMAX_INT8)
    return dequant_token_group_bf16(int_dot_groups(q_a, w_q, group_size), s2[:, 0], s_w), q_a, s2[:, 0]


def w8a8_linear_token_group(x: np.ndarray, w_q: np.ndarray, s_w: np.ndarray, group_size: int):
    """Per-token activation codes (one scale per row of x) against per-group
    weight codes (group_size 64 or 128 along K). Returns (y, q_a, s_a)."""
    q_a, s_a = quantize_act(x, 0)
    y = dequant_token_group(int_dot_groups(q_a, w_q, group_size), s_a, s_w)
    return y, q_a, s_a
