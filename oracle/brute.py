"""Exact-arithmetic brute force of the same method, for tiny inputs.

TEST INFRASTRUCTURE, like the rest of this folder: only tests, the smoke
check and the benchmark's CPU-baseline leg may use it.

It shares no arithmetic with the numpy oracle. Every value is a Python
Fraction; fp32 and fp16 results are produced by an explicit
round-to-nearest-even routine written here from the IEEE 754 definition (p
significand bits, minimum normal exponent emin, gradual underflow), and the
integer accumulation uses Python ints. The method's steps are the ones of the
Cider README's kernel pipeline and quantization sections (per-token or
per-group symmetric min-max codes, int32 accumulation, dequant as
acc * s_act * s_weight rounded to fp16); the readings of the unstated details
(scale = max|v| / qmax in fp32, ties to even, a zero group gets scale 0) are
the same ones the numpy oracle documents.
"""
from __future__ import annotations

from fractions import Fraction

__all__ = ["round_binary", "f32", "f16", "f64", "bf16", "linear_bf16", "rint_half_even", "quantize_row", "percentile_fp64",
           "quantize_row_clip",
           "dot", "dequant", "dequant_groups", "linear", "mv", "linear_token_group"]

_INF = float("inf")


def round_binary(v: Fraction, p: int, emin: int, emax: int):
    """Round v to the nearest binary floating-point number with p significand
    bits (hidden bit included), exponents in [emin, emax], subnormals below
    2**emin; ties go to the even significand. Returns a Fraction, or +-inf
    when the rounded magnitude reaches 2**(emax+1)."""
    v = Fraction(v)
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = -v if v < 0 else v
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2**(e-1) < a < 2**(e+1); settle e with 2**e <= a < 2**(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)                       # subnormal range shares emin's ulp
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        return sign * _INF
    return sign * r


def f32(v) -> Fraction:
    return round_binary(Fraction(v), 24, -126, 127)


def f16(v) -> Fraction:
    return round_binary(Fraction(v), 11, -14, 15)


def bf16(v) -> Fraction:
    """bfloat16: 8 significand bits, the exponent range of fp32."""
    return round_binary(Fraction(v), 8, -126, 127)


def f64(v) -> Fraction:
    return round_binary(Fraction(v), 53, -1022, 1023)


def rint_half_even(v: Fraction) -> int:
    fl = v.numerator // v.denominator
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def quantize_row(values, group_size: int, qmax: int):
    """values: exact fp16 values of one row (floats or Fractions).
    Returns (codes list[int], scales list[Fraction]) with one scale per group."""
    vals = [Fraction(v) for v in values]
    K = len(vals)
    gs = K if group_size == 0 else group_size
    assert K % gs == 0
    codes, scales = [], []
    for g in range(K // gs):
        grp = vals[g * gs:(g + 1) * gs]
        amax = max(abs(v) for v in grp)
        s = f32(amax / qmax)
        scales.append(s)
        for v in grp:
            if s == 0:
                codes.append(0)
            else:
                c = rint_half_even(f32(v / s))
                codes.append(max(-qmax, min(qmax, c)))
    return codes, scales


def percentile_fp64(mags, percentile: float) -> Fraction:
    """The clip threshold of one group: position h = (n-1) * (p/100), value
    a[i] + (h - i) * (a[j] - a[i]) over the ascending magnitudes, each step
    rounded to fp64 as written, then the result rounded to fp32."""
    a = sorted(Fraction(m) for m in mags)
    n = len(a)
    h = f64(Fraction(n - 1) * f64(Fraction(percentile) / 100))
    i = h.numerator // h.denominator
    j = min(i + 1, n - 1)
    g = h - i
    return f32(f64(a[i] + f64(g * (a[j] - a[i]))))


def quantize_row_clip(values, group_size: int, qmax: int, percentile: float):
    """quantize_row with s = t / qmax, t = percentile_fp64 of the group."""
    vals = [Fraction(v) for v in values]
    K = len(vals)
    gs = K if group_size == 0 else group_size
    codes, scales = [], []
    for g in range(K // gs):
        grp = vals[g * gs:(g + 1) * gs]
        s = f32(percentile_fp64([abs(v) for v in grp], percentile) / qmax)
        scales.append(s)
        for v in grp:
            codes.append(0 if s == 0 else max(-qmax, min(qmax, rint_half_even(f32(v / s)))))
    return codes, scales


def dot(a, b) -> int:
    return sum(int(x) * int(y) for x, y in zip(a, b))


def dequant(acc: int, s_a: Fraction, s_w: Fraction) -> Fraction:
    return f16(Fraction(acc) * s_a * s_w)


def dequant_groups(accs, s_as, s_ws) -> Fraction:
    return f16(sum(Fraction(c) * a * w for c, a, w in zip(accs, s_as, s_ws)))


def linear(x_rows, w_codes, w_scales, group_size: int):
    """x_rows: list of fp16-valued rows; w_codes: list of int code rows [N][K];
    w_scales: per row, a list of G scales (Fractions). Returns
    (y [M][N] Fractions, qa [M][K], sa [M][G])."""
    K = len(x_rows[0]) if x_rows else 0
    gs = K if group_size == 0 else group_size
    qa, sa = [], []
    for row in x_rows:
        c, s = quantize_row(row, group_size, 127)
        qa.append(c)
        sa.append(s)
    y = []
    for m in range(len(x_rows)):
        out = []
        for n in range(len(w_codes)):
            accs = [dot(qa[m][g * gs:(g + 1) * gs], w_codes[n][g * gs:(g + 1) * gs])
                    for g in range(K // gs)]
            out.append(dequant_groups(accs, sa[m], w_scales[n]))
        y.append(out)
    return y, qa, sa


def linear_bf16(x_rows, w_codes, w_scales, group_size: int):
    """linear() with the output rounded once to bfloat16 instead of fp16 (the
    activation rows are bf16 values; the quantization steps are the same)."""
    K = len(x_rows[0]) if x_rows else 0
    gs = K if group_size == 0 else group_size
    qa, sa = [], []
    for row in x_rows:
        c, s = quantize_row(row, group_size, 127)
        qa.append(c)
        sa.append(s)
    y = []
    for m in range(len(x_rows)):
        out = []
        for n in range(len(w_codes)):
            accs = [dot(qa[m][g * gs:(g + 1) * gs], w_codes[n][g * gs:(g + 1) * gs]) for g in range(K // gs)]
            out.append(bf16(sum(Fraction(c) * a * w for c, a, w in zip(accs, sa[m], w_scales[n]))))
        y.append(out)
    return y, qa, sa


def mv(x_rows, w_codes, w_scales, group_size: int):
    """Decode MV (README kernel pipeline, Decode: int8_mv; no activation
    quantization): y[m][n] = f16( sum_k x[m][k] * code[n][k] * scale[n][g(k)] ),
    the sum exact. x_rows: fp16-valued numbers; w_codes: int rows; w_scales:
    per row a list of G scale Fractions."""
    K = len(x_rows[0]) if x_rows else 0
    gs = K if group_size == 0 else group_size
    y = []
    for row in x_rows:
        out = []
        for codes, scales in zip(w_codes, w_scales):
            t = sum(Fraction(row[k]) * int(codes[k]) * scales[k // gs] for k in range(K))
            out.append(f16(t))
        y.append(out)
    return y


def linear_token_group(x_rows, w_codes, w_scales, group_size: int, out=None):
    """Per-token activation codes (one scale per row) against per-group weight
    codes: y[m][n] = f16( sum_g acc_g * s_a[m] * s_w[n][g] ), exact; `out`
    rounds the exact sum instead (bf16 for a bfloat16 output)."""
    out_round = f16 if out is None else out
    K = len(x_rows[0]) if x_rows else 0
    y = []
    for row in x_rows:
        c, s = quantize_row(row, 0, 127)
        out = []
        for n in range(len(w_codes)):
            t = sum(Fraction(dot(c[g * group_size:(g + 1) * group_size],
                                 w_codes[n][g * group_size:(g + 1) * group_size])) * s[0] * w_scales[n][g]
                    for g in range(K // group_size))
            out.append(out_round(t))
        y.append(out)
    return y
