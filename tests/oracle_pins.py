"""Checks that pin the CPU oracle to facts fixed outside itself.

Each check takes an implementation namespace with the oracle's functions
(the primitives quantize_rows, pack_int4, unpack_int4, int_dot,
int_dot_groups, the dequants, int8_mv, the percentile and bf16 helpers, and
the composite entry points built from them) and raises AssertionError when
the implementation disagrees with:

* hand-derived worked examples stored under tests/golden/ (closed forms);
* the exact-rational brute force in oracle/brute.py on tiny inputs;
* invariants of the definition (2^k scaling, sign symmetry, range, K
  permutation, gs = K reducing to per-channel);
* the deterministic error bound of symmetric min-max quantization against the
  unquantized fp64 product, and cosine floors on the synthetic workload;
* the composition of the primitives, for every composite entry point.

The same checks run against deliberately broken copies of the oracle in
test_oracle_mutants.py, to show that each plausible mistake is caught.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _act(impl, x, gs):
    q, s = impl.quantize_rows(x, gs, 127)
    return q, s


def _linear(impl, x, wq, sw2d, gs):
    """Compose the primitives into the W8A8 linear; sw2d is [N, G]."""
    qa, sa = impl.quantize_rows(x, gs, 127)
    if gs == 0:
        return impl.dequant_per_channel(impl.int_dot(qa, wq), sa[:, 0], sw2d[:, 0])
    return impl.dequant_per_group(impl.int_dot_groups(qa, wq, gs), sa, sw2d)


# --------------------------------------------------------------- golden files
def check_golden_quant(impl):
    for case in _load("quant_ties.json")["cases"]:
        x = np.array([case["x"]], np.float16)
        q, s = impl.quantize_rows(x, case["group_size"], case["qmax"])
        assert q.tolist()[0] == case["q"], (case, q)
        assert s.astype(np.float64).ravel().tolist() == case["s"], (case, s)


def check_golden_division(impl):
    """Rows where only a correctly rounded fp32 division by the scale (not a
    multiplication by its rounded reciprocal) gives the right code."""
    for case in _load("division_cases.json")["cases"]:
        x = np.array([case["x"]], np.float16)
        q, s = impl.quantize_rows(x, 0, 127)
        assert q.tolist()[0] == case["q"], (case, q)
        assert float(s[0, 0]) == case["s"], (case, s)


def check_golden_int4(impl):
    g = _load("int4_pack.json")
    codes = np.array(g["codes"], np.int8)
    packed = impl.pack_int4(codes)
    assert packed.dtype == np.uint8 and packed.tolist() == g["packed"], packed
    assert impl.unpack_int4(np.array(g["packed"], np.uint8)).tolist() == g["codes"]


def check_golden_integer_gemm(impl):
    g = _load("integer_gemm.json")
    x = np.array(g["x"], np.float16)
    w = np.array(g["w"], np.float16)
    qa, sa = impl.quantize_rows(x, 0, 127)
    qw, sw = impl.quantize_rows(w, 0, 127)
    assert np.all(sa == 1) and np.all(sw == 1)
    acc = impl.int_dot(qa, qw)
    assert acc.tolist() == g["acc"], acc
    y = impl.dequant_per_channel(acc, sa[:, 0], sw[:, 0])
    assert y.astype(np.float64).tolist() == g["y"], y


def check_closed_form_k10240(impl):
    g = _load("closed_form_k10240.json")
    K = g["K"]
    x = np.full((2, K), g["x_value"], np.float16)
    w = np.full((2, K), g["w_value"], np.float16)
    w[1, K // 3] = g["w_special_value"]
    qa, sa = impl.quantize_rows(x, 0, 127)
    qw, sw = impl.quantize_rows(w, 0, 127)
    assert np.all(qa == 127) and np.all(sa == np.float32(2.0 ** -20))
    assert np.all(sw == np.float32(2.0 ** -10)) and qw[1, K // 3] == 1
    acc = impl.int_dot(qa, qw)
    assert acc[0, 0] == g["acc_all_127"] and acc[0, 1] == g["acc_one_code_1"], acc
    y = impl.dequant_per_channel(acc, sa[:, 0], sw[:, 0])
    assert float(y[0, 1]) == g["y_one_code_1"], y


# --------------------------------------------------------------- brute force
def _rand_fp16(rng, shape, kind):
    if kind == "normal":
        v = rng.standard_normal(shape) * 3
    elif kind == "wide":
        v = rng.standard_normal(shape) * np.exp2(rng.integers(-12, 12, size=shape))
    elif kind == "ties":      # values that land on code midpoints when amax = 127
        v = rng.integers(-254, 255, size=shape) / 2.0
        v.flat[0] = 127.0
    else:
        v = rng.integers(-3, 4, size=shape).astype(np.float64)
    return v.astype(np.float16)


def check_brute_quant(impl, trials=60, seed=1):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        R = int(rng.integers(1, 5))
        gs = [0, 2, 4][t % 3]
        K = int(rng.integers(1, 3)) * 4
        qmax = 127 if t % 4 else 7
        x = _rand_fp16(rng, (R, K), ["normal", "wide", "ties", "small"][t % 4])
        q, s = impl.quantize_rows(x, gs, qmax)
        for r in range(R):
            bq, bs = brute.quantize_row([float(v) for v in x[r]], gs, qmax)
            assert q[r].tolist() == bq, (x[r], q[r], bq)
            assert [Fraction(float(v)) for v in s[r]] == bs, (x[r], s[r], bs)


def check_brute_linear(impl, trials=24, seed=2):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [0, 4, 8][t % 3]
        K = 16 if gs else int(rng.integers(1, 9)) * 2
        x = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3])
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "small"][t % 3])
        qw, sw = impl.quantize_rows(w, gs, 127)
        with np.errstate(over="ignore"):   # fp16 overflow to inf is the IEEE reading
            y = _linear(impl, x, qw, sw, gs)
        wcodes = qw.astype(int).tolist()
        wsc = [[Fraction(float(v)) for v in row] for row in sw]
        by, bqa, bsa = brute.linear([[float(v) for v in row] for row in x], wcodes, wsc, gs)
        for m in range(M):
            for n in range(N):
                assert float(y[m, n]) == float(by[m][n]), (t, m, n, y[m, n], float(by[m][n]))
        # the int32 accumulators, one group at a time
        qa, _ = impl.quantize_rows(x, gs, 127)
        accg = impl.int_dot_groups(qa, qw, gs)
        g_sz = K if gs == 0 else gs
        for g in range(accg.shape[0]):
            for m in range(M):
                for n in range(N):
                    ref = brute.dot(bqa[m][g * g_sz:(g + 1) * g_sz], wcodes[n][g * g_sz:(g + 1) * g_sz])
                    assert accg[g, m, n] == ref


def check_brute_int4(impl, trials=20, seed=3):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        N, K = int(rng.integers(1, 4)), int(rng.integers(1, 5)) * 2
        w = _rand_fp16(rng, (N, K), "normal")
        q, s = impl.quantize_rows(w, 0, 7)
        p = impl.pack_int4(q)
        for n in range(N):
            bq, bs = brute.quantize_row([float(v) for v in w[n]], 0, 7)
            assert q[n].tolist() == bq
            by = [(bq[2 * j] + 8) | ((bq[2 * j + 1] + 8) << 4) for j in range(K // 2)]
            assert p[n].tolist() == by
        assert np.array_equal(impl.unpack_int4(p), q)


# --------------------------------------------------------------- invariants
def check_pow2_invariance(impl, seed=4):
    """Scaling a row by 2^k (exactly representable) keeps the codes and
    multiplies the scale by exactly 2^k."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6, 256)) * 4).astype(np.float16)
    x[:, 7] *= np.float16(16)
    for gs in (0, 64, 128):
        q0, s0 = impl.quantize_rows(x, gs, 127)
        for k in range(-3, 9):
            xs = (x.astype(np.float64) * 2.0 ** k).astype(np.float16)
            exact = (xs.astype(np.float64) * 2.0 ** -k == x.astype(np.float64)).all(axis=1)
            q1, s1 = impl.quantize_rows(xs, gs, 127)
            for r in np.nonzero(exact)[0]:
                assert np.array_equal(q1[r], q0[r]), (gs, k, r)
                assert np.array_equal(s1[r], (s0[r].astype(np.float64) * 2.0 ** k).astype(np.float32))


def check_sign_and_range(impl, seed=5):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((16, 128)) * 10).astype(np.float16)
    for qmax in (127, 7):
        for gs in (0, 64):
            q, s = impl.quantize_rows(x, gs, qmax)
            qn, sn = impl.quantize_rows(-x, gs, qmax)
            assert np.array_equal(qn, -q) and np.array_equal(sn, s)
            assert np.abs(q.astype(int)).max() <= qmax
            G = s.shape[1]
            gsz = 128 // G
            xr = np.abs(x.astype(np.float32)).reshape(16, G, gsz)
            qr = q.reshape(16, G, gsz)
            at = xr.argmax(axis=2)
            picked = np.take_along_axis(qr, at[:, :, None], axis=2)[:, :, 0]
            assert np.all(np.abs(picked.astype(int)) == qmax)
    z = np.zeros((2, 64), np.float16)
    q, s = impl.quantize_rows(z, 0, 127)
    assert not q.any() and not s.any()


def check_k_permutation(impl, seed=6):
    rng = np.random.default_rng(seed)
    qa = rng.integers(-127, 128, (5, 96)).astype(np.int8)
    qw = rng.integers(-127, 128, (7, 96)).astype(np.int8)
    perm = rng.permutation(96)
    a = impl.int_dot(qa, qw)
    assert np.array_equal(a, impl.int_dot(qa[:, perm], qw[:, perm]))
    ref = qa.astype(np.int64) @ qw.astype(np.int64).T
    assert np.array_equal(a, ref)
    assert a.shape == (5, 7)


def check_gs_equals_k(impl, seed=7):
    """Per-group with one group spanning all of K is per-channel."""
    rng = np.random.default_rng(seed)
    for K in (64, 128):
        x = (rng.standard_normal((9, K)) * 2).astype(np.float16)
        w = (rng.standard_normal((11, K)) * 0.02).astype(np.float16)
        qw, sw = impl.quantize_rows(w, 0, 127)
        qwg, swg = impl.quantize_rows(w, K, 127)
        assert np.array_equal(qw, qwg) and np.array_equal(sw, swg)
        y0 = _linear(impl, x, qw, sw, 0)
        y1 = _linear(impl, x, qwg, swg, K)
        assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))


def error_bound(x, w, qa, sa, qw, sw, gs_a, gs_w):
    """Deterministic bound on |y - x W^T| for symmetric round-to-nearest codes.

    With x = s_a*q_a + e_a and |e_a| <= (s_a/2)(1 + 2^-15) (the rint of a
    correctly rounded quotient of magnitude <= 128), and likewise for W:
    x W - (s_a q_a)(s_w q_w) = x e_w + e_a W - e_a e_w, and the fp16 rounding
    of the output adds 2^-11 relative plus half the smallest subnormal."""
    K = x.shape[1]
    ga = K if gs_a == 0 else gs_a
    gw = K if gs_w == 0 else gs_w
    sa_k = np.repeat(sa.astype(np.float64), ga, axis=1)  # [M, K]
    sw_k = np.repeat(sw.astype(np.float64), gw, axis=1)  # [N, K]
    ax = np.abs(x.astype(np.float64))
    aw = np.abs(w.astype(np.float64))
    c = (1 + 2.0 ** -15) ** 2
    bq = c * (ax @ (sw_k / 2).T + (sa_k / 2) @ aw.T + (sa_k / 2) @ (sw_k / 2).T)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    return ref, bq + 2.0 ** -11 * (np.abs(ref) + bq) + 2.0 ** -24 + 1e-12 * (ax @ aw.T)


def cosine(a, b):
    a = a.astype(np.float64).ravel()
    b = b.astype(np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b) + 1e-12))


def check_error_bound_and_cosine(impl, M=48, N=96, seed=0):
    from w8a8_online_quantized_amd import inputs
    for K, gs, floor in ((2560, 0, 0.997), (10240, 0, 0.997), (1024, 128, 0.999), (1024, 64, 0.999)):
        x = inputs.activations(M, K, seed=seed)
        w = inputs.weights(N, K, seed=seed)
        qw, sw = impl.quantize_rows(w, gs, 127)
        qa, sa = impl.quantize_rows(x, gs, 127)
        y = _linear(impl, x, qw, sw, gs)
        ref, bound = error_bound(x, w, qa, sa, qw, sw, gs, gs)
        err = np.abs(y.astype(np.float64) - ref)
        assert np.all(err <= bound), (K, gs, float((err - bound).max()))
        cs = cosine(y, ref)
        assert cs >= floor, (K, gs, cs)


def check_int4_bound_and_cosine(impl, M=48, N=96, seed=0):
    from w8a8_online_quantized_amd import inputs
    K = 2560
    x = inputs.activations(M, K, seed=seed)
    w = inputs.weights(N, K, seed=seed)
    q4, s4 = impl.quantize_rows(w, 0, 7)
    qw = impl.unpack_int4(impl.pack_int4(q4))
    qa, sa = impl.quantize_rows(x, 0, 127)
    y = impl.dequant_per_channel(impl.int_dot(qa, qw), sa[:, 0], s4[:, 0])
    ref, bound = error_bound(x, w, qa, sa, qw, s4, 0, 0)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err - bound).max())
    assert cosine(y, ref) >= 0.98



# ------------------------------------------------------------------ decode MV
def check_golden_mv(impl):
    for c in _load("int8_mv.json")["cases"]:
        x = np.array(c["x"], np.float16)
        y = impl.int8_mv(x, np.array(c["w_q"], np.int8), np.array(c["s_w"], np.float32), c["group_size"])
        assert y.tolist() == c["y"], (c["name"], y.tolist(), c["y"])


def check_brute_mv(impl, trials=30, seed=11):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [0, 2, 4, 8][t % 4]
        K = 8 * int(rng.integers(1, 3)) if gs else int(rng.integers(1, 12))
        x = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3])
        G = 1 if gs == 0 else K // gs
        q = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
        sw = (np.abs(rng.standard_normal((N, G))) * 2.0 ** rng.integers(-12, 2, size=(N, G))).astype(np.float32)
        with np.errstate(over="ignore"):
            y = impl.int8_mv(x, q, sw, gs)
        by = brute.mv([[float(v) for v in row] for row in x], q.astype(int).tolist(),
                      [[Fraction(float(v)) for v in row] for row in sw], gs)
        for m in range(M):
            for n in range(N):
                assert float(y[m, n]) == float(by[m][n]), (t, m, n, y[m, n], float(by[m][n]))


def check_mv_gs_equals_k(impl, seed=12):
    rng = np.random.default_rng(seed)
    K = 128
    x = (rng.standard_normal((3, K)) * 2).astype(np.float16)
    q = rng.integers(-127, 128, size=(7, K)).astype(np.int8)
    sw = (np.abs(rng.standard_normal((7, 1))) * 1e-2).astype(np.float32)
    y0 = impl.int8_mv(x, q, sw, 0)
    y1 = impl.int8_mv(x, q, sw, K)
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))


def check_mv_pow2_scaling(impl, seed=13):
    """Scaling x by 2^k scales y by 2^k exactly (no overflow / underflow here)."""
    rng = np.random.default_rng(seed)
    K = 64
    x = (rng.standard_normal((4, K))).astype(np.float16)
    q = rng.integers(-127, 128, size=(9, K)).astype(np.int8)
    for gs in (0, 32):
        G = 1 if gs == 0 else K // gs
        sw = (np.abs(rng.standard_normal((9, G))) * 1e-2 + 1e-3).astype(np.float32)
        y = impl.int8_mv(x, q, sw, gs).astype(np.float64)
        for k in (-2, 1, 3):
            y2 = impl.int8_mv((x.astype(np.float32) * 2.0 ** k).astype(np.float16), q, sw, gs).astype(np.float64)
            ok = np.abs(y) >= 2.0 ** -12
            assert np.array_equal(y2[ok], y[ok] * 2.0 ** k), (gs, k)


def check_mv_matches_lossless_w8a8(impl, seed=14):
    """On activations that per-token quantization reproduces exactly (each row
    is codes * 2^-3 with some |code| = 127, so s_a = 2^-3 and the codes come
    back unchanged), the decode MV and the W8A8 linear compute the same exact
    value acc * s_a * s_w, so their fp16 outputs agree bit for bit."""
    rng = np.random.default_rng(seed)
    K, N = 256, 40
    codes = rng.integers(-127, 128, size=(5, K))
    codes[:, 7] = 127
    x = (codes * 0.125).astype(np.float16)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    qw, sw = impl.quantize_rows(w, 0, 127)
    qa, sa = impl.quantize_rows(x, 0, 127)
    assert np.array_equal(qa, codes.astype(np.int8)) and np.all(sa == 0.125)
    y8 = _linear(impl, x, qw, sw, 0)
    ymv = impl.int8_mv(x, qw, sw, 0)
    assert np.array_equal(y8.view(np.uint16), ymv.view(np.uint16))


def check_mv_exact_sum(impl, trials=12, seed=15):
    """Large cancelling products next to tiny ones. Every product x*q is a
    multiple of 2^-24 below 2^22, so with K = 64 every partial sum fits the
    53-bit fp64 significand exactly, in any order: the oracle must return the
    exact sum rounded once (the brute force), which an fp32 running sum loses."""
    rng = np.random.default_rng(seed)
    K = 64
    for t in range(trials):
        x = (rng.uniform(0.5, 1.0, (2, K)) * 2.0 ** rng.integers(-14, -6, size=(2, K))).astype(np.float64)
        q = rng.integers(-127, 128, size=(3, K)).astype(np.int8)
        for i, j in ((0, K - 1), (2 + t % 7, 40 + t % 11), (20, 21)):
            big = float(2 ** 14 + 2 ** rng.integers(0, 10))
            x[:, i], x[:, j] = big, -big
            q[:, j] = q[:, i]
        x = x.astype(np.float16)
        sw = np.full((3, 1), 2.0 ** -8, np.float32)
        y = impl.int8_mv(x, q, sw, 0)
        by = brute.mv([[float(v) for v in row] for row in x], q.astype(int).tolist(),
                      [[Fraction(float(v)) for v in row] for row in sw], 0)
        for m in range(2):
            for n in range(3):
                assert float(y[m, n]) == float(by[m][n]), (t, m, n, float(y[m, n]), float(by[m][n]))


# ------------------------------------------------- per-token x per-group weight
def check_golden_token_group(impl):
    for c in _load("token_group.json")["cases"]:
        x = np.array(c["x"], np.float16)
        qa, sa = impl.quantize_rows(x, 0, 127)
        assert qa.tolist() == c["q_a"] and sa[:, 0].tolist() == c["s_a"]
        wq = np.array(c["w_q"], np.int8)
        y = impl.dequant_token_group(impl.int_dot_groups(qa, wq, c["group_size"]), sa[:, 0],
                                     np.array(c["s_w"], np.float32))
        assert y.tolist() == c["y"], (y.tolist(), c["y"])


def check_brute_token_group(impl, trials=20, seed=16):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [2, 4, 8][t % 3]
        K = gs * int(rng.integers(1, 4))
        x = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3])
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "small"][t % 3])
        qw, sw = impl.quantize_rows(w, gs, 127)
        qa, sa = impl.quantize_rows(x, 0, 127)
        with np.errstate(over="ignore"):
            y = impl.dequant_token_group(impl.int_dot_groups(qa, qw, gs), sa[:, 0], sw)
        by = brute.linear_token_group([[float(v) for v in row] for row in x], qw.astype(int).tolist(),
                                      [[Fraction(float(v)) for v in row] for row in sw], gs)
        for m in range(M):
            for n in range(N):
                assert float(y[m, n]) == float(by[m][n]), (t, m, n, y[m, n], float(by[m][n]))


def check_token_group_reductions(impl, seed=17):
    """One group spanning K is per-channel; activations whose groups all have
    the same max|x| make per-group activation codes equal the per-token ones,
    and then per-group and per-token x per-group coincide bit for bit."""
    rng = np.random.default_rng(seed)
    K, gs = 256, 64
    x = (rng.standard_normal((6, K)) * 2).astype(np.float16)
    w = (rng.standard_normal((9, K)) * 0.02).astype(np.float16)
    qa, sa = impl.quantize_rows(x, 0, 127)
    qw0, sw0 = impl.quantize_rows(w, 0, 127)
    y0 = impl.dequant_per_channel(impl.int_dot(qa, qw0), sa[:, 0], sw0[:, 0])
    y1 = impl.dequant_token_group(impl.int_dot_groups(qa, qw0, K), sa[:, 0], sw0)
    assert np.array_equal(y0.view(np.uint16), y1.view(np.uint16))
    x[:, ::gs] = np.float16(8.0)          # every group of every row: max|x| = 8
    qa, sa = impl.quantize_rows(x, 0, 127)
    qag, sag = impl.quantize_rows(x, gs, 127)
    assert np.array_equal(qa, qag) and np.all(sag == sa)
    qw, sw = impl.quantize_rows(w, gs, 127)
    acc = impl.int_dot_groups(qa, qw, gs)
    y2 = impl.dequant_per_group(acc, sag, sw)
    y3 = impl.dequant_token_group(acc, sa[:, 0], sw)
    assert np.array_equal(y2.view(np.uint16), y3.view(np.uint16))

# ------------------------------------------------- percentile-clipped weight scales
def check_golden_clip(impl):
    for c in _load("clip_percentile.json")["cases"]:
        x = np.array([c["x"]], np.float16)
        t = impl.percentile_threshold(np.abs(x.astype(np.float32)), c["percentile"])
        assert float(t[0]) == c["t"], (c["percentile"], float(t[0]), c["t"])
        q, s = impl.quantize_rows_clip(x, 0, c["qmax"], c["percentile"])
        assert float(s[0, 0]) == float(np.float32(c["t"]) / np.float32(c["qmax"]))
        assert q[0].tolist() == c["q"], (c["percentile"], q[0].tolist())


def check_brute_clip(impl, trials=48, seed=18):
    """Exact-rational brute force (its own rounding routines) on tiny groups."""
    rng = np.random.default_rng(seed)
    ps = [0.0, 12.5, 50.0, 90.0, 99.0, 99.9, 100.0]
    for t in range(trials):
        gs = [0, 2, 4, 8][t % 4]
        K = (gs or 1) * int(rng.integers(1, 5)) if gs else int(rng.integers(1, 13))
        x = _rand_fp16(rng, (2, K), ["normal", "wide", "ties", "small"][t % 4])
        p = ps[t % len(ps)] if t < 2 * len(ps) else float(rng.uniform(0, 100))
        qmax = 127 if t % 3 else 7
        q, sc = impl.quantize_rows_clip(x, gs, qmax, p)
        for r in range(2):
            bq, bs = brute.quantize_row_clip([float(v) for v in x[r]], gs, qmax, p)
            assert q[r].tolist() == bq, (t, r, p, q[r].tolist(), bq)
            assert [float(v) for v in sc[r]] == [float(v) for v in bs], (t, r, p)


def check_clip_vs_numpy_percentile(impl, seed=19):
    """The threshold against numpy.percentile (default method, computed in
    fp64 by numpy's own code): within one fp32 ulp."""
    rng = np.random.default_rng(seed)
    for n in (64, 128, 1000, 2560, 10240):
        m = np.abs(rng.standard_normal((6, n)).astype(np.float16)).astype(np.float32)
        m[0, :: 97] *= np.float32(30)
        for p in (99.9, 99.0, 95.0, 50.0, 1.0, 100.0, 33.3):
            t = impl.percentile_threshold(m, p)
            ref = np.percentile(m.astype(np.float64), p, axis=-1).astype(np.float32)
            ulp = np.spacing(np.abs(ref))
            assert np.all(np.abs(t.astype(np.float64) - ref) <= ulp), (n, p, t, ref)


def check_clip_reductions(impl, seed=20):
    """Percentile 100 is min-max bit for bit; constant magnitudes make every
    percentile min-max; a lone outlier is clipped (saturated code, smaller
    scale, smaller error elsewhere); the threshold grows with the percentile."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((8, 256)) * 0.05).astype(np.float16)
    for gs in (0, 64):
        for qmax in (127, 7):
            q1, s1 = impl.quantize_rows_clip(w, gs, qmax, 100.0)
            q0, s0 = impl.quantize_rows(w, gs, qmax)
            assert np.array_equal(q1, q0) and np.array_equal(s1, s0)
    c = np.where(rng.random((4, 128)) < 0.5, np.float16(-0.75), np.float16(0.75)).astype(np.float16)
    for p in (0.0, 37.5, 99.9):
        qc, sc = impl.quantize_rows_clip(c, 0, 127, p)
        q0, s0 = impl.quantize_rows(c, 0, 127)
        assert np.array_equal(qc, q0) and np.array_equal(sc, s0)
    K = 2560
    row = (rng.standard_normal((1, K)) * 0.02).astype(np.float16)
    big = int(rng.integers(0, K))
    row[0, big] = np.float16(np.abs(row.astype(np.float32)).max() * 50)
    qc, sc = impl.quantize_rows_clip(row, 0, 127, 99.9)
    q0, s0 = impl.quantize_rows(row, 0, 127)
    assert sc[0, 0] < s0[0, 0] / 10 and abs(int(qc[0, big])) == 127
    v = row[0].astype(np.float64)
    keep = np.ones(K, bool)
    keep[big] = False
    tval = float(impl.percentile_threshold(np.abs(row.astype(np.float32)), 99.9)[0])
    inside = keep & (np.abs(v) <= tval)
    err_c = np.abs(v - float(sc[0, 0]) * qc[0].astype(np.float64))
    err_0 = np.abs(v - float(s0[0, 0]) * q0[0].astype(np.float64))
    assert np.all(err_c[inside] <= float(sc[0, 0]) * (0.5 + 1e-6))
    assert err_c[keep].mean() < err_0[keep].mean() / 5
    m = np.abs(rng.standard_normal((3, 512)).astype(np.float16)).astype(np.float32)
    ts = [impl.percentile_threshold(m, p) for p in (10.0, 50.0, 90.0, 99.0, 99.9, 100.0)]
    for a, b in zip(ts, ts[1:]):
        assert np.all(a <= b)
    assert np.array_equal(ts[-1], m.max(axis=-1))


# ------------------------------------------------- bf16 I/O
def _bf16_bits(h):
    return np.array([int(h, 16)], np.uint16)


def check_golden_bf16(impl):
    d = _load("bf16.json")
    for c in d["round"]:
        got = int(impl.f64_to_bf16(np.array([c["v"]]))[0])
        assert got == int(c["bits"], 16), (c, hex(got))
        got = int(impl.f64_to_bf16(np.array([-c["v"]]))[0])
        assert got == int(c["bits"], 16) ^ 0x8000, (c, "negated", hex(got))
    for c in d["decode"]:
        v = float(impl.bf16_to_f32(_bf16_bits(c["bits"]))[0])
        assert v == float(c["v"]), (c, v)


def check_brute_bf16_rounding(impl, seed=21):
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(1500) * 10.0 ** rng.integers(-44, 39, 1500)
    v = np.concatenate([v, rng.integers(-300, 300, 200) * 2.0 ** rng.integers(-140, 120, 200)])
    got = impl.f64_to_bf16(v)
    for x, b in zip(v, got):
        ref = brute.bf16(Fraction(float(x)))
        val = float(impl.bf16_to_f32(np.array([b], np.uint16))[0])
        assert val == float(ref), (x, val, float(ref))


def check_brute_linear_bf16(impl, trials=24, seed=22):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [0, 2, 4][t % 3]
        K = (gs or 1) * int(rng.integers(1, 5)) if gs else int(rng.integers(1, 9))
        xf = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3]).astype(np.float32)
        xb = (xf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)      # truncated to bf16
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "small"][t % 3])
        qw, sw = impl.quantize_rows(w, gs, 127)
        qa, sa = impl.quantize_rows_bf16(xb, gs, 127)
        acc = impl.int_dot(qa, qw) if gs == 0 else impl.int_dot_groups(qa, qw, gs)
        y = impl.dequant_bf16(acc, sa[:, 0] if gs == 0 else sa, sw[:, 0] if gs == 0 else sw)
        xr = [[float(v) for v in row] for row in impl.bf16_to_f32(xb)]
        by, bq, _ = brute.linear_bf16(xr, qw.astype(int).tolist(), [[Fraction(float(v)) for v in row] for row in sw], gs)
        assert qa.astype(int).tolist() == bq, t
        yv = impl.bf16_to_f32(y)
        for m in range(M):
            for n in range(N):
                assert float(yv[m, n]) == float(by[m][n]), (t, m, n, float(yv[m, n]), float(by[m][n]))


def check_brute_token_group_bf16(impl, trials=18, seed=24):
    """bf16 rows in, per-token codes against per-group weight codes, bf16 out,
    against the exact-arithmetic reference rounded once to bf16."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [2, 4, 8][t % 3]
        K = gs * int(rng.integers(1, 4))
        xf = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3]).astype(np.float32)
        xb = (xf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)      # truncated to bf16
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "small"][t % 3])
        qw, sw = impl.quantize_rows(w, gs, 127)
        qa, sa = impl.quantize_rows_bf16(xb, 0, 127)
        y = impl.dequant_token_group_bf16(impl.int_dot_groups(qa, qw, gs), sa[:, 0], sw)
        xr = [[float(v) for v in row] for row in impl.bf16_to_f32(xb)]
        by = brute.linear_token_group(xr, qw.astype(int).tolist(), [[Fraction(float(v)) for v in row] for row in sw],
                                      gs, out=brute.bf16)
        yv = impl.bf16_to_f32(y)
        for m in range(M):
            for n in range(N):
                assert float(yv[m, n]) == float(by[m][n]), (t, m, n, float(yv[m, n]), float(by[m][n]))


def check_bf16_reductions(impl, seed=23):
    """bf16 rows whose values are fp16 values too quantize exactly as the fp16
    rows do; a bf16 output equals the fp16 output wherever the exact value
    fits both formats."""
    rng = np.random.default_rng(seed)
    xf = (rng.integers(-255, 256, (6, 128)) * 2.0 ** rng.integers(-8, 4, (6, 1))).astype(np.float32)
    xb = (xf.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    assert np.array_equal(impl.bf16_to_f32(xb), xf)
    for gs in (0, 64):
        q1, s1 = impl.quantize_rows_bf16(xb, gs, 127)
        q0, s0 = impl.quantize_rows(xf.astype(np.float16), gs, 127)
        assert np.array_equal(q1, q0) and np.array_equal(s1, s0)
    acc = rng.integers(-2 ** 14, 2 ** 14, (5, 7))
    s_a = np.full(5, 2.0 ** -6, np.float32)
    s_w = np.full(7, 2.0 ** -3, np.float32)
    yb = impl.dequant_bf16(acc, s_a, s_w)
    small = np.abs(acc) < 256                 # acc * 2^-9 has at most 8 significant bits
    y16 = impl.dequant_per_channel(acc, s_a, s_w)
    assert np.array_equal(impl.bf16_to_f32(yb)[small], y16.astype(np.float32)[small])


# ------------------------------------------------- long K: exact single rounding
def _double_rounding_cases(count=4):
    """Per-channel (acc, s_a, s_w) whose exact product lies 2^-63 above or below
    a midpoint of fp16 while the fp64 product acc * s_a rounds onto that
    midpoint: acc * m = H +- 1 with H = (2j+1) * 2^43 (an fp16 midpoint once
    scaled by 2^-63), s_a = m * 2^-23 (m odd, 24 bits), s_w = 2^-40, |acc| near
    2^31 (K well past 33k). Pure integer search: m must divide H +- 1, and
    2j+1 is taken 1 mod 4 for +1 (3 mod 4 for -1) so that the exact value's
    side of the midpoint is away from the even neighbour."""
    out = []
    for sign in (1, -1):
        m = 2 ** 23 + 1
        while len([c for c in out if c[3] == sign]) < count // 2:
            inv = pow(2 ** 43, -1, m)
            r = (-sign * inv) % m          # (2j+1) * 2^43 + sign == 0 (mod m)
            if r % 4 == (1 if sign > 0 else 3) and 2 ** 11 <= r < 2 ** 12:
                h = r * 2 ** 43
                acc = (h + sign) // m
                if acc < 2 ** 31:
                    out.append((acc, m, h, sign))
            m += 2
    return out


def check_dequant_long_k_exact(impl):
    """|acc| near 2^31 (reachable for K up to the library's limit): the
    per-channel dequant is the exact product rounded once, also where the
    fp64 product acc * s_a is inexact and rounds onto an fp16 midpoint, so a
    second rounding of it would go to the even neighbour whatever the side
    the exact value lies on."""
    cases = _double_rounding_cases()
    sw_list = []
    for acc_i, m, h, sign in cases:
        sa = np.float32(m * 2.0 ** -23)
        assert float(sa) == m * 2.0 ** -23                      # exactly representable
        v = impl.dequant_per_channel(np.array([[acc_i]], np.int64), np.array([sa], np.float32),
                                     np.array([2.0 ** -40], np.float32))
        exact = brute.f16(Fraction(acc_i) * Fraction(float(sa)) * Fraction(2) ** -40)
        assert float(v[0, 0]) == float(exact), (acc_i, m, sign, float(v[0, 0]), float(exact))
        naive = np.float16((np.float64(acc_i) * np.float64(sa)) * 2.0 ** -40)
        sw_list.append(float(naive) != float(exact))
    assert all(sw_list), "a case did not exercise a double rounding"
    # random accumulators up to the int32 limit against the brute force
    rng = np.random.default_rng(31)
    acc = rng.integers(-(2 ** 31) + 1, 2 ** 31, (6, 7))
    s_a = (rng.uniform(1, 2, 6) * 2.0 ** rng.integers(-20, -6, 6)).astype(np.float32)
    s_w = (rng.uniform(1, 2, 7) * 2.0 ** rng.integers(-12, -4, 7)).astype(np.float32)
    with np.errstate(over="ignore"):
        y = impl.dequant_per_channel(acc, s_a, s_w)
    for m in range(6):
        for n in range(7):
            ref = brute.f16(Fraction(int(acc[m, n])) * Fraction(float(s_a[m])) * Fraction(float(s_w[n])))
            assert float(y[m, n]) == float(ref), (m, n, float(y[m, n]), float(ref))


# ------------------------------------------------- composite entry points
# The public composites (weight quantizers, bf16 and per-token x per-group
# linears) must equal their composition of the primitives pinned above, bit
# for bit, and the exact-rational brute force on tiny shapes.
def _pack_ref(codes):
    """Two codes per byte, the even K index (plus 8) in the low nibble."""
    return [(codes[2 * j] + 8) | ((codes[2 * j + 1] + 8) << 4) for j in range(len(codes) // 2)]


def _unpack_ref(row):
    out = []
    for b in row:
        out += [(int(b) & 15) - 8, (int(b) >> 4) - 8]
    return out


def _to_bf16_bits(xf):
    """fp32 values that are bf16 values -> their uint16 patterns (exact)."""
    return (np.asarray(xf, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def check_weight_quantizers_compose(impl, seed=40):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((6, 128)) * 0.05).astype(np.float16)
    w[2, 17] = np.float16(1.5)                                   # an outlier to clip
    wb = _to_bf16_bits(w.astype(np.float32))                    # fp16 values with <= 8 bits? not always
    wb_vals = impl.bf16_to_f32(wb)
    for gs in (0, 64):
        q, s = impl.quantize_weight(w, 8, gs)
        q0, s0 = impl.quantize_rows(w, gs, 127)
        assert np.array_equal(q, q0) and np.array_equal(s.reshape(6, -1), s0)
        for p in (99.9, 50.0):
            q, s = impl.quantize_weight_clip(w, 8, gs, p)
            q0, s0 = impl.quantize_rows_clip(w, gs, 127, p)
            assert np.array_equal(q, q0) and np.array_equal(s.reshape(6, -1), s0), (gs, p)
        q, s = impl.quantize_weight_bf16(wb, 8, gs)
        q0, s0 = impl.quantize_rows_bf16(wb, gs, 127)
        assert np.array_equal(q, q0) and np.array_equal(s.reshape(6, -1), s0)
    q, s = impl.quantize_weight(w, 4, 0)
    q0, s0 = impl.quantize_rows(w, 0, 7)
    assert np.array_equal(q, impl.pack_int4(q0)) and np.array_equal(s, s0[:, 0])
    q, s = impl.quantize_weight_clip(w, 4, 0, 99.0)
    q0, s0 = impl.quantize_rows_clip(w, 0, 7, 99.0)
    assert q.shape == (6, 64) and np.array_equal(q, impl.pack_int4(q0)) and np.array_equal(s, s0[:, 0])
    q, s = impl.quantize_weight_bf16(wb, 4, 0)
    q0, s0 = impl.quantize_rows_bf16(wb, 0, 7)
    assert np.array_equal(q, impl.pack_int4(q0)) and np.array_equal(s, s0[:, 0])
    # bf16 rows whose values are also fp16 values: the bf16 clip quantizer is
    # the fp16 one on the same values
    exact16 = np.all(wb_vals.astype(np.float16).astype(np.float32) == wb_vals, axis=1)
    assert exact16.any()
    rows = np.nonzero(exact16)[0]
    for bits, gs in ((8, 0), (8, 64), (4, 0)):
        q, s = impl.quantize_weight_clip_bf16(wb[rows], bits, gs, 90.0)
        q0, s0 = impl.quantize_weight_clip(wb_vals[rows].astype(np.float16), bits, gs, 90.0)
        assert np.array_equal(q, q0) and np.array_equal(s, s0), (bits, gs)


def check_weight_quantizers_brute(impl, trials=24, seed=41):
    """Every weight quantizer against the exact-rational brute force and the
    nibble layout written out here."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        bits = 8 if t % 2 else 4
        gs = 0 if bits == 4 else [0, 2, 4][t % 3]
        K = (gs or 2) * int(rng.integers(1, 4))
        N = int(rng.integers(1, 4))
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "ties", "small"][t % 4])
        wf = w.astype(np.float32)
        wb = _to_bf16_bits(wf)                                    # truncation: a bf16 value
        wbf = impl.bf16_to_f32(wb)
        p = [99.9, 50.0, 0.0, 75.0][t % 4]
        qmax = 127 if bits == 8 else 7
        for fn, vals, args in ((impl.quantize_weight, wf, ()), (impl.quantize_weight_clip, wf, (p,)),
                               (impl.quantize_weight_bf16, wbf, ()), (impl.quantize_weight_clip_bf16, wbf, (p,))):
            src = w if fn in (impl.quantize_weight, impl.quantize_weight_clip) else wb
            q, s = fn(src, bits, gs, *args)
            s2 = np.asarray(s).reshape(N, -1)
            for n in range(N):
                row = [float(v) for v in vals[n]]
                if args:
                    bq, bs = brute.quantize_row_clip(row, gs, qmax, p)
                else:
                    bq, bs = brute.quantize_row(row, gs, qmax)
                got = q[n].tolist()
                want = _pack_ref(bq) if bits == 4 else bq
                assert got == want, (fn.__name__, t, n, got, want)
                assert [float(v) for v in s2[n]] == [float(v) for v in bs], (fn.__name__, t, n)


def check_linear_composites_compose(impl, seed=42):
    """The linears equal their primitive compositions bit for bit."""
    from w8a8_online_quantized_amd import inputs
    x = inputs.activations(8, 256, seed=seed)
    w = inputs.weights(12, 256, seed=seed)
    xb = _to_bf16_bits(x.astype(np.float32))
    for gs in (0, 64, 128):
        wq, sw = impl.quantize_weight(w, 8, gs)
        sw2 = sw[:, None] if gs == 0 else sw
        y, qa, sa = impl.w8a8_linear(x, wq, sw, gs)
        assert np.array_equal(y.view(np.uint16), _linear(impl, x, wq, sw2, gs).view(np.uint16)), gs
        yb, qb, sb = impl.w8a8_linear_bf16(xb, wq, sw, gs)
        q0, s0 = impl.quantize_rows_bf16(xb, gs, 127)
        assert np.array_equal(qb, q0) and np.array_equal(np.asarray(sb).reshape(8, -1), s0), gs
        acc = impl.int_dot(q0, wq) if gs == 0 else impl.int_dot_groups(q0, wq, gs)
        want = impl.dequant_bf16(acc, s0[:, 0] if gs == 0 else s0, sw)
        assert np.array_equal(yb, want), gs
    p, s4 = impl.quantize_weight(w, 4, 0)
    y4, _, _ = impl.w4a8_linear(x, p, s4)
    y8, _, _ = impl.w8a8_linear(x, impl.unpack_int4(p), s4, 0)
    assert np.array_equal(y4.view(np.uint16), y8.view(np.uint16))
    y4b, q4b, s4b = impl.w4a8_linear_bf16(xb, p, s4)
    y8b, _, _ = impl.w8a8_linear_bf16(xb, impl.unpack_int4(p), s4, 0)
    assert np.array_equal(y4b, y8b)
    for gs in (64, 128):
        wq, sw = impl.quantize_weight(w, 8, gs)
        y, qa, sa = impl.w8a8_linear_token_group(x, wq, sw, gs)
        q0, s0 = impl.quantize_rows(x, 0, 127)
        assert np.array_equal(qa, q0) and np.array_equal(sa, s0[:, 0])
        want = impl.dequant_token_group(impl.int_dot_groups(q0, wq, gs), s0[:, 0], sw)
        assert np.array_equal(y.view(np.uint16), want.view(np.uint16)), gs
        yb, qb, sb = impl.w8a8_linear_token_group_bf16(xb, wq, sw, gs)
        q0, s0 = impl.quantize_rows_bf16(xb, 0, 127)
        assert np.array_equal(qb, q0) and np.array_equal(sb, s0[:, 0])
        assert np.array_equal(yb, impl.dequant_token_group_bf16(impl.int_dot_groups(q0, wq, gs), s0[:, 0], sw)), gs


def check_linear_composites_brute(impl, trials=18, seed=43):
    """bf16, W4A8-bf16 and per-token x per-group linears against the brute force."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        gs = [2, 4][t % 2]
        K = 4 * int(rng.integers(1, 4))
        x = _rand_fp16(rng, (M, K), ["normal", "wide", "ties"][t % 3])
        xb = _to_bf16_bits(x.astype(np.float32))
        xr = [[float(v) for v in row] for row in impl.bf16_to_f32(xb)]
        x16 = [[float(v) for v in row] for row in x]
        w = _rand_fp16(rng, (N, K), ["normal", "wide", "small"][t % 3])
        # per-token x per-group, fp16 and bf16
        wq, sw = impl.quantize_rows(w, gs, 127)
        wc = wq.astype(int).tolist()
        wsc = [[Fraction(float(v)) for v in row] for row in sw]
        with np.errstate(over="ignore"):
            y, qa, _ = impl.w8a8_linear_token_group(x, wq, sw, gs)
        by = brute.linear_token_group(x16, wc, wsc, gs)
        assert [[float(v) for v in r] for r in y] == [[float(v) for v in r] for r in by], ("tok", t)
        yb, _, _ = impl.w8a8_linear_token_group_bf16(xb, wq, sw, gs)
        byb = brute.linear_token_group(xr, wc, wsc, gs, out=brute.bf16)
        assert impl.bf16_to_f32(yb).tolist() == [[float(v) for v in r] for r in byb], ("tok bf16", t)
        # bf16 linear (per-group codes along the same groups)
        yb, qb, _ = impl.w8a8_linear_bf16(xb, wq, sw, gs)
        byb, bq, _ = brute.linear_bf16(xr, wc, wsc, gs)
        assert qb.astype(int).tolist() == bq
        assert impl.bf16_to_f32(yb).tolist() == [[float(v) for v in r] for r in byb], ("bf16", t)
        # W4A8 with bf16 rows: the packed bytes unpacked by the layout written here
        q4, s4 = impl.quantize_rows(w, 0, 7)
        p = impl.pack_int4(q4)
        yb, _, _ = impl.w4a8_linear_bf16(xb, p, s4[:, 0])
        codes = [_unpack_ref(row) for row in p.tolist()]
        byb, _, _ = brute.linear_bf16(xr, codes, [[Fraction(float(r[0]))] for r in s4], 0)
        assert impl.bf16_to_f32(yb).tolist() == [[float(v) for v in r] for r in byb], ("w4a8 bf16", t)


ALL_CHECKS = [
    check_golden_quant, check_golden_division, check_golden_int4, check_golden_integer_gemm,
    check_closed_form_k10240, check_brute_quant, check_brute_linear,
    check_brute_int4, check_pow2_invariance, check_sign_and_range,
    check_k_permutation, check_gs_equals_k, check_error_bound_and_cosine,
    check_int4_bound_and_cosine, check_golden_mv, check_brute_mv, check_mv_gs_equals_k,
    check_mv_pow2_scaling, check_mv_matches_lossless_w8a8, check_mv_exact_sum,
    check_golden_token_group, check_brute_token_group, check_token_group_reductions,
    check_golden_clip, check_brute_clip, check_clip_vs_numpy_percentile, check_clip_reductions,
    check_golden_bf16, check_brute_bf16_rounding, check_brute_linear_bf16, check_bf16_reductions,
    check_brute_token_group_bf16, check_dequant_long_k_exact, check_weight_quantizers_compose,
    check_weight_quantizers_brute, check_linear_composites_compose, check_linear_composites_brute,
]
