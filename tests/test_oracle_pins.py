"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something other than its own formula:
exact rational arithmetic, closed forms, brute force over tiny inputs, a
library routine that computes the same definition another way, or an
invariant.  The cases are chosen so that a plausible slip in the oracle (a
dropped term, a wrong scale index, a transposed operand, a wrong rounding
mode, mean vs sum, a sign) fails at least one of them.
"""
import itertools
import math
import os
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_q8(rng, n_out, n_in):
    return synthetic.q8_matrix(rng, n_out, n_in)


# ---------------------------------------------------------------------------
# G: f32-activation GEMV


@pytest.mark.parametrize("n_out,n_in,m", [(3, 64, 1), (4, 96, 2), (5, 32, 3)])
def test_gemv_f32_matches_exact_rational(n_out, n_in, m):
    rng = np.random.default_rng(11)
    Wq, Ws = _rand_q8(rng, n_out, n_in)
    x = synthetic.normal(rng, m, n_in)
    y = oracle.gemv_f32(Wq, Ws, x)
    for r in range(m):
        for o in range(n_out):
            terms = [Fraction(int(Wq[o, t])) * Fraction(float(Ws[o, t // 32])) * Fraction(float(x[r, t]))
                     for t in range(n_in)]
            exact = sum(terms, Fraction(0))
            mag = float(sum(abs(t) for t in terms))
            assert abs(Fraction(y[r, o]) - exact) <= Fraction((n_in + 1) * mag) * Fraction(2) ** -52


def test_gemv_f32_equals_dense_dequant_matmul():
    rng = np.random.default_rng(12)
    Wq, Ws = _rand_q8(rng, 37, 320)
    x = synthetic.normal(rng, 3, 320)
    W = Wq.astype(np.float64) * np.repeat(Ws.astype(np.float64), 32, axis=1)
    ref = x.astype(np.float64) @ W.T
    y = oracle.gemv_f32(Wq, Ws, x)
    assert np.max(np.abs(y - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_gemv_f32_scale_index_is_per_block_of_32():
    # Wq = 1, x = 1, distinct power-of-two scale per (row, block):
    # y[o] = 32 * sum_b Ws[o, b].  A t%32 (instead of t/32) index, or a
    # transposed scale table, gives a different sum.
    n_out, n_in = 3, 128
    Wq = np.ones((n_out, n_in), np.int8)
    Ws = np.array([[2.0 ** -(o * 4 + b) for b in range(4)] for o in range(n_out)], np.float32)
    x = np.ones((1, n_in), np.float32)
    y = oracle.gemv_f32(Wq, Ws, x)[0]
    for o in range(n_out):
        assert y[o] == 32 * sum(2.0 ** -(o * 4 + b) for b in range(4))


def test_gemv_f32_rows_are_outputs():
    # A weight with one non-zero row picks out exactly that output.
    Wq = np.zeros((4, 64), np.int8)
    Wq[2, 5] = -7
    Ws = np.ones((4, 2), np.float32)
    x = np.arange(64, dtype=np.float32)[None, :]
    y = oracle.gemv_f32(Wq, Ws, x)[0]
    assert list(y) == [0.0, 0.0, -35.0, 0.0]


def test_gemv_f32_fill_closed_forms():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "fill_closed_forms.txt")) if l.strip() and not l.startswith("#")]
    assert rows
    for n_in, s, expect in rows:
        n_in, s, expect = int(n_in), float(s), float(expect)
        Wq = np.ones((2, n_in), np.int8)
        Ws = np.full((2, n_in // 32), s, np.float32)
        x = synthetic.fill_pattern(n_in)[None, :]
        y = oracle.gemv_f32(Wq, Ws, x)[0]
        assert list(y) == [expect, expect]


def test_gemv_f32_linear_in_power_of_two_factors():
    rng = np.random.default_rng(13)
    Wq, Ws = _rand_q8(rng, 8, 64)
    x = synthetic.normal(rng, 1, 64)
    z = synthetic.normal(rng, 1, 64)
    y1 = oracle.gemv_f32(Wq, Ws, 4.0 * x)
    assert np.array_equal(y1, 4.0 * oracle.gemv_f32(Wq, Ws, x))
    yx, yz, ys = oracle.gemv_f32(Wq, Ws, x), oracle.gemv_f32(Wq, Ws, z), oracle.gemv_f32(Wq, Ws, x + z)
    # x + z is rounded to f32, so linearity holds to the f32 rounding of the sum
    assert np.max(np.abs(ys - (yx + yz))) <= 1e-6 * np.max(np.abs(ys))


# ---------------------------------------------------------------------------
# Q: the Q8_0 activation quantiser


def _nearest_away(p):
    """Brute force: of the 255 codes -127..127, the one nearest to the float p,
    ties away from zero."""
    best = None
    for c in range(-127, 128):
        dist = abs(Fraction(c) - Fraction(float(p)))
        if best is None or dist < best[0] or (dist == best[0] and abs(c) > abs(best[1])):
            best = (dist, c)
    return best[1]


def test_quantize_brute_force():
    rng = np.random.default_rng(21)
    v = np.concatenate([synthetic.normal(rng, 2, 64), 1e-3 * synthetic.normal(rng, 1, 64),
                        np.round(synthetic.normal(rng, 1, 64) * 20) / 4], axis=0).astype(np.float32)
    q, d = oracle.quantize(v)
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            blk = v[r, b * 32:(b + 1) * 32]
            amax = np.float32(np.max(np.abs(blk)))
            dd = np.float32(amax) / np.float32(127.0)
            assert d[r, b] == dd
            idv = np.float32(1.0) / dd if dd != 0 else np.float32(0.0)
            for t in range(32):
                p = np.float32(blk[t]) * np.float32(idv)
                assert q[r, b * 32 + t] == _nearest_away(p), (r, b, t)


def test_quantize_closed_forms():
    # A block of integers holding +-127 has d = 1 and q = v.
    blk = np.array([127, -127] + list(range(-15, 15)), np.float32)
    q, d = oracle.quantize(blk[None, :])
    assert d[0, 0] == 1.0 and np.array_equal(q[0].astype(np.float32), blk)
    # A zero block: d = 0, q = 0.
    q, d = oracle.quantize(np.zeros((1, 32), np.float32))
    assert d[0, 0] == 0.0 and not q.any()
    # Halfway cases round away from zero (amax 127 gives d = 1, id = 1).
    blk = np.zeros(32, np.float32)
    blk[:7] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -126.5]
    q, d = oracle.quantize(blk[None, :])
    assert list(q[0, :7]) == [127, 3, -3, 1, -1, 2, -127]


def test_quantize_round_trip_bound():
    rng = np.random.default_rng(22)
    v = synthetic.normal(rng, 8, 256)
    q, d = oracle.quantize(v)
    back = q.astype(np.float64) * np.repeat(d.astype(np.float64), 32, axis=1)
    bound = np.repeat(d.astype(np.float64), 32, axis=1) * (0.5 + 1e-5)
    assert np.all(np.abs(back - v) <= bound)
    assert np.all(np.abs(q) <= 127)


# ---------------------------------------------------------------------------
# exact int32 block dots, and I: the int8-activation GEMV


def test_block_dots_brute_force_and_extremes():
    rng = np.random.default_rng(31)
    Wq = synthetic.quants(rng, 3, 64)
    xq = synthetic.quants(rng, 2, 64)
    isum = oracle.block_dots(Wq, xq)
    for r in range(2):
        for o in range(3):
            for b in range(2):
                s = sum(int(Wq[o, t]) * int(xq[r, t]) for t in range(b * 32, b * 32 + 32))
                assert isum[r, o, b] == s
    W = np.full((1, 32), 127, np.int8)
    X = np.full((1, 32), -127, np.int8)
    assert oracle.block_dots(W, X)[0, 0, 0] == -516128


def test_gemv_i8_exact_special_case():
    # Power-of-two scales and the (p % 7) - 3 fill make every float step exact.
    n_out, n_in = 6, 128
    Wq = (synthetic.fill_pattern(n_out * n_in).reshape(n_out, n_in)).astype(np.int8)
    xq = synthetic.fill_pattern(n_in + 3)[3:].astype(np.int8)[None, :]
    Ws = np.array([[2.0 ** -((o + b) % 5) for b in range(4)] for o in range(n_out)], np.float32)
    xs = np.array([[2.0 ** -(b % 3) for b in range(4)]], np.float32)
    y = oracle.gemv_i8(Wq, Ws, xq, xs)[0]
    for o in range(n_out):
        exact = sum(Fraction(float(Ws[o, b])) * Fraction(float(xs[0, b])) *
                    sum(int(Wq[o, t]) * int(xq[0, t]) for t in range(32 * b, 32 * b + 32)) for b in range(4))
        assert Fraction(y[o]) == exact


def test_gemv_i8_matches_exact_rational():
    rng = np.random.default_rng(32)
    Wq, Ws = _rand_q8(rng, 4, 96)
    x = synthetic.normal(rng, 2, 96)
    xq, xs = oracle.quantize(x)
    y = oracle.gemv_i8(Wq, Ws, xq, xs)
    for r in range(2):
        for o in range(4):
            terms = [Fraction(float(Ws[o, b])) * Fraction(float(xs[r, b])) *
                     sum(int(Wq[o, t]) * int(xq[r, t]) for t in range(32 * b, 32 * b + 32)) for b in range(3)]
            exact = sum(terms, Fraction(0))
            mag = float(sum(abs(t) for t in terms))
            assert abs(Fraction(y[r, o]) - exact) <= Fraction(8 * mag) * Fraction(2) ** -52


def test_gemv_i8_within_quantisation_bound_of_f32_mode():
    rng = np.random.default_rng(33)
    Wq, Ws = _rand_q8(rng, 64, 256)
    x = synthetic.normal(rng, 2, 256)
    xq, xs = oracle.quantize(x)
    yi = oracle.gemv_i8(Wq, Ws, xq, xs)
    yf = oracle.gemv_f32(Wq, Ws, x)
    Wabs = np.abs(Wq.astype(np.float64)) * np.repeat(Ws.astype(np.float64), 32, axis=1)
    bound = Wabs @ (np.repeat(xs.astype(np.float64), 32, axis=1) * 0.50001).T
    assert np.all(np.abs(yi - yf) <= bound.T + 1e-12)


# ---------------------------------------------------------------------------
# Q2 and I2: the two-word (~14-bit) activation and its GEMV.  The pages give
# the words, the low words and one scale a block (arena.rs fn quant_parts);
# the low word's weight of 1/128 of a step is the reading pinned here.


def _low_word_brute_force(p, q):
    """Of the 255 low words -127..127, the one whose lo/128 is nearest to the
    exact rest p - q, ties away from zero."""
    rest = Fraction(float(p)) - q
    best = None
    for c in range(-127, 128):
        dist = abs(Fraction(c, 128) - rest)
        if best is None or dist < best[0] or (dist == best[0] and abs(c) > abs(best[1])):
            best = (dist, c)
    return best[1]


def test_quantize_x2_words_and_scales_are_one_word():
    rng = np.random.default_rng(41)
    v = synthetic.normal(rng, 4, 128)
    q, lo, d = oracle.quantize_x2(v)
    q1, d1 = oracle.quantize(v)
    assert np.array_equal(q, q1) and np.array_equal(d, d1)


def test_quantize_x2_low_words_brute_force():
    rng = np.random.default_rng(42)
    v = np.concatenate([synthetic.normal(rng, 2, 64), 1e-3 * synthetic.normal(rng, 1, 64)], axis=0)
    q, lo, d = oracle.quantize_x2(v)
    assert np.max(np.abs(lo.astype(int))) <= 64
    for r in range(v.shape[0]):
        for b in range(v.shape[1] // 32):
            idv = np.float32(1.0) / d[r, b] if d[r, b] != 0 else np.float32(0.0)
            for t in range(b * 32, b * 32 + 32):
                p = np.float32(v[r, t]) * np.float32(idv)
                assert lo[r, t] == _low_word_brute_force(p, int(q[r, t])), (r, t)


def test_quantize_x2_closed_forms():
    # amax 127 gives d = 1, id = 1: the rest after the word is exact
    blk = np.zeros(32, np.float32)
    vals = [127.0, 3.25, -2.75, 2.5, -2.5, 0.75, 1.0 + 1.0 / 256, -1.0 / 512, 5.0 + 63.0 / 128]
    blk[:len(vals)] = vals
    q, lo, d = oracle.quantize_x2(blk[None, :])
    assert d[0, 0] == 1.0
    assert list(q[0, :len(vals)]) == [127, 3, -3, 3, -3, 1, 1, 0, 5]
    assert list(lo[0, :len(vals)]) == [0, 32, 32, -64, 64, -32, 1, 0, 63]
    # a zero block: scale, words and low words all zero
    q, lo, d = oracle.quantize_x2(np.zeros((1, 32), np.float32))
    assert d[0, 0] == 0.0 and not q.any() and not lo.any()


def test_quantize_x2_reconstruction_bound():
    rng = np.random.default_rng(43)
    v = synthetic.normal(rng, 8, 256).astype(np.float64)
    q, lo, d = oracle.quantize_x2(v.astype(np.float32))
    dd = np.repeat(d.astype(np.float64), 32, axis=1)
    back = dd * (q.astype(np.float64) + lo.astype(np.float64) / 128.0)
    # half a 128th of a step, plus the float32 rounding of v * id
    assert np.all(np.abs(back - v) <= dd / 256.0 + np.abs(v) * 2.0 ** -22)
    q1, d1 = oracle.quantize(v.astype(np.float32))
    err1 = np.abs(q1.astype(np.float64) * dd - v)
    assert np.mean(np.abs(back - v)) < np.mean(err1) / 32.0


def test_gemv_i8x2_matches_exact_rational():
    rng = np.random.default_rng(44)
    Wq, Ws = _rand_q8(rng, 4, 96)
    x = synthetic.normal(rng, 2, 96)
    xq, xl, xs = oracle.quantize_x2(x)
    y = oracle.gemv_i8x2(Wq, Ws, xq, xl, xs)
    for r in range(2):
        for o in range(4):
            terms = [Fraction(float(Ws[o, b])) * Fraction(float(xs[r, b])) *
                     sum(int(Wq[o, t]) * (Fraction(int(xq[r, t])) + Fraction(int(xl[r, t]), 128))
                         for t in range(32 * b, 32 * b + 32)) for b in range(3)]
            exact = sum(terms, Fraction(0))
            mag = float(sum(abs(t) for t in terms))
            assert abs(Fraction(y[r, o]) - exact) <= Fraction(8 * mag) * Fraction(2) ** -52


def test_gemv_i8x2_without_low_words_is_one_word():
    rng = np.random.default_rng(45)
    Wq, Ws = _rand_q8(rng, 16, 128)
    xq, xs = oracle.quantize(synthetic.normal(rng, 3, 128))
    y1 = oracle.gemv_i8(Wq, Ws, xq, xs)
    y2 = oracle.gemv_i8x2(Wq, Ws, xq, np.zeros_like(xq), xs)
    assert np.array_equal(y1, y2)


def test_gemv_i8x2_equals_f32_mode_on_exact_rows():
    # rows that the two words represent exactly: power-of-two block scales,
    # one word of 127 a block (so the block's amax gives back its scale), low
    # words of at most 63 (so the word is the rounding of the value)
    rng = np.random.default_rng(46)
    m, n = 3, 160
    q = rng.integers(-126, 127, size=(m, n)).astype(np.int64)
    lo = rng.integers(-63, 64, size=(m, n)).astype(np.int64)
    q[:, ::32] = 127
    lo[:, ::32] = 0
    d = (2.0 ** rng.integers(-9, -2, size=(m, n // 32))).astype(np.float32)
    x = (np.repeat(d.astype(np.float64), 32, axis=1) * (q + lo / 128.0)).astype(np.float32)
    xq, xl, xs = oracle.quantize_x2(x)
    assert np.array_equal(xs, d) and np.array_equal(xq, q.astype(np.int8)) and np.array_equal(xl, lo.astype(np.int8))
    Wq, Ws = _rand_q8(rng, 24, n)
    y2 = oracle.gemv_i8x2(Wq, Ws, xq, xl, xs)
    yf = oracle.gemv_f32(Wq, Ws, x)
    assert np.max(np.abs(y2 - yf)) <= 1e-12 * np.max(np.abs(yf))


def test_gemv_i8x2_within_quantisation_bound_of_f32_mode():
    rng = np.random.default_rng(47)
    Wq, Ws = _rand_q8(rng, 64, 256)
    x = synthetic.normal(rng, 2, 256)
    xq, xl, xs = oracle.quantize_x2(x)
    y2 = oracle.gemv_i8x2(Wq, Ws, xq, xl, xs)
    yf = oracle.gemv_f32(Wq, Ws, x)
    Wabs = np.abs(Wq.astype(np.float64)) * np.repeat(Ws.astype(np.float64), 32, axis=1)
    step = np.repeat(xs.astype(np.float64), 32, axis=1) / 256.0 + np.abs(x.astype(np.float64)) * 2.0 ** -22
    bound = Wabs @ step.T
    assert np.all(np.abs(y2 - yf) <= bound.T + 1e-12)
    # and far inside the one-word bound
    xq1, xs1 = oracle.quantize(x)
    y1 = oracle.gemv_i8(Wq, Ws, xq1, xs1)
    assert np.max(np.abs(y2 - yf)) < np.max(np.abs(y1 - yf)) / 16.0


# ---------------------------------------------------------------------------
# N: residual add + RMSNorm


def test_add_rmsnorm_sum_is_f32_add():
    rng = np.random.default_rng(41)
    h, r = synthetic.normal(rng, 3, 96), synthetic.normal(rng, 3, 96)
    w = rng.uniform(0.5, 1.5, 96).astype(np.float32)
    s, _ = oracle.add_rmsnorm(h, r, w, 1e-6)
    assert np.array_equal(s, (h + r).astype(np.float32))


def test_add_rmsnorm_constant_row_closed_form():
    d, c, eps = 64, 0.75, 1e-6
    h = np.full((1, d), c, np.float32)
    r = np.zeros((1, d), np.float32)
    w = np.linspace(0.5, 1.5, d).astype(np.float32)
    _, y = oracle.add_rmsnorm(h, r, w, eps)
    ref = w.astype(np.float64) * c / math.sqrt(c * c + np.float64(np.float32(eps)))
    assert np.max(np.abs(y[0] - ref)) <= 1e-15


def test_add_rmsnorm_matches_high_precision():
    getcontext().prec = 60
    rng = np.random.default_rng(42)
    d = 96
    h, r = synthetic.normal(rng, 2, d), synthetic.normal(rng, 2, d)
    w = rng.uniform(0.5, 1.5, d).astype(np.float32)
    eps = np.float32(1e-5)
    s, y = oracle.add_rmsnorm(h, r, w, eps)
    for i in range(2):
        ms = sum(Fraction(float(v)) ** 2 for v in s[i]) / d
        den = (Decimal(ms.numerator) / Decimal(ms.denominator) + Decimal(float(eps))).sqrt()
        for t in range(d):
            ref = Decimal(float(s[i, t])) * Decimal(float(w[t])) / den
            # ss carries up to ~d ulps of rounding; sqrt halves it.  A slip in the
            # formula (sum for mean, eps outside the root) is >= 1e-6 relative.
            assert abs(Decimal(y[i, t]) - ref) <= Decimal(4e-15) * abs(ref) + Decimal(1e-300)


def test_add_rmsnorm_fused_equals_unfused():
    # add then norm with no residual gives the same result as the fused call
    rng = np.random.default_rng(43)
    h, r = synthetic.normal(rng, 2, 128), synthetic.normal(rng, 2, 128)
    w = rng.uniform(0.5, 1.5, 128).astype(np.float32)
    s, y = oracle.add_rmsnorm(h, r, w, 1e-6)
    s2, y2 = oracle.add_rmsnorm((h + r).astype(np.float32), np.zeros_like(h), w, 1e-6)
    assert np.array_equal(s, s2) and np.array_equal(y, y2)


# ---------------------------------------------------------------------------
# R: routing


@pytest.mark.parametrize("E,k", [(6, 2), (8, 3), (10, 4), (5, 5)])
def test_route_brute_force_over_subsets(E, k):
    rng = np.random.default_rng(51 + E)
    d = 64
    Wr = (0.02 * synthetic.normal(rng, E, d)).astype(np.float32)
    x = synthetic.normal(rng, 3, d)
    idx, wts, logits = oracle.route(x, Wr, k)
    for i in range(3):
        l = [sum(Fraction(float(Wr[e, t])) * Fraction(float(x[i, t])) for t in range(d)) for e in range(E)]
        # the kept set maximises the summed logit; among equal sums, the
        # lexicographically smallest index set
        best = max(itertools.combinations(range(E), k), key=lambda c: (sum(l[e] for e in c), [-e for e in c]))
        assert sorted(idx[i]) == list(best)
        # rank order: logit descending, index ascending
        order = sorted(best, key=lambda e: (-l[e], e))
        assert list(idx[i]) == order
        # weights: softmax over E, kept, renormalised (scipy's softmax)
        p = scipy.special.softmax(np.array([float(v) for v in l]))
        ref = p[order] / p[order].sum()
        assert np.max(np.abs(wts[i] - ref)) <= 1e-14
        assert abs(wts[i].sum() - 1.0) <= 1e-12


def test_route_logits_are_router_matvec():
    rng = np.random.default_rng(52)
    Wr = (0.02 * synthetic.normal(rng, 128, 256)).astype(np.float32)
    x = synthetic.normal(rng, 4, 256)
    _, _, logits = oracle.route(x, Wr, 8)
    ref = x.astype(np.float64) @ Wr.astype(np.float64).T
    assert np.max(np.abs(logits - ref)) <= 1e-13 * np.max(np.abs(ref))


def test_route_degenerate_cases():
    d = 64
    x = synthetic.normal(np.random.default_rng(53), 1, d)
    # a zero router: every logit 0, ties to the lower index, equal weights
    idx, wts, _ = oracle.route(x, np.zeros((16, d), np.float32), 4)
    assert list(idx[0]) == [0, 1, 2, 3] and np.allclose(wts[0], 0.25, rtol=0, atol=1e-15)
    # K = 1 gives weight 1
    Wr = (0.02 * synthetic.normal(np.random.default_rng(54), 16, d)).astype(np.float32)
    idx, wts, l = oracle.route(x, Wr, 1)
    assert wts[0, 0] == 1.0 and idx[0, 0] == int(np.argmax(l[0]))
    # explicit ties: rows 3 and 1 equal and largest -> 1 ranks before 3
    Wr2 = np.zeros((6, d), np.float32)
    Wr2[3] = Wr2[1] = x[0] / 8
    Wr2[5] = x[0] / 16
    idx, wts, _ = oracle.route(x, Wr2, 3)
    assert list(idx[0]) == [1, 3, 5]
    assert wts[0, 0] == wts[0, 1] > wts[0, 2]


# ---------------------------------------------------------------------------
# R8: routing over Q8_0 router rows


@pytest.mark.parametrize("E,k", [(6, 2), (8, 3), (9, 4)])
def test_route_q8_brute_force_over_subsets(E, k):
    # float activations: the exact rational logits of the dequantised rows,
    # the kept set the best-summed subset, the weights scipy's softmax
    rng = np.random.default_rng(61 + E)
    d = 64
    Wq, Ws = _rand_q8(rng, E, d)
    x = synthetic.normal(rng, 2, d)
    idx, wts, logits = oracle.route_q8(Wq, Ws, k, x=x)
    for i in range(2):
        l = [sum(Fraction(int(Wq[e, t])) * Fraction(float(Ws[e, t // 32])) * Fraction(float(x[i, t]))
                 for t in range(d)) for e in range(E)]
        assert np.max(np.abs(logits[i] - np.array([float(v) for v in l]))) <= 1e-14 * max(abs(float(v)) for v in l)
        best = max(itertools.combinations(range(E), k), key=lambda c: (sum(l[e] for e in c), [-e for e in c]))
        order = sorted(best, key=lambda e: (-l[e], e))
        assert list(idx[i]) == order
        p = scipy.special.softmax(np.array([float(v) for v in l]))
        assert np.max(np.abs(wts[i] - p[order] / p[order].sum())) <= 1e-14


def test_route_q8_int8_logits_brute_force():
    # int8 activations: per 32-value block, the exact integer dot of the two
    # quantised rows times both scales, summed (exact rationals)
    rng = np.random.default_rng(64)
    E, d, k = 7, 96, 3
    Wq, Ws = _rand_q8(rng, E, d)
    xq = rng.integers(-127, 128, size=(2, d)).astype(np.int8)
    xs = (rng.random((2, d // 32)) * 0.05 + 0.001).astype(np.float32)
    idx, wts, logits = oracle.route_q8(Wq, Ws, k, xq=xq, xs=xs)
    for i in range(2):
        l = []
        for e in range(E):
            acc = Fraction(0)
            for b in range(d // 32):
                dot = sum(int(Wq[e, t]) * int(xq[i, t]) for t in range(32 * b, 32 * b + 32))
                acc += Fraction(float(Ws[e, b])) * Fraction(float(xs[i, b])) * dot
            l.append(acc)
        assert np.max(np.abs(logits[i] - np.array([float(v) for v in l]))) <= 1e-14 * max(abs(float(v)) for v in l)
        assert list(idx[i]) == sorted(range(E), key=lambda e: (-l[e], e))[:k]


def test_route_q8_equals_float_router_on_exact_rows():
    # power-of-two scales: every dequantised weight is an exact float32, so
    # routing over the Q8_0 rows equals routing over those float32 rows
    rng = np.random.default_rng(65)
    E, d, k = 64, 256, 6
    Wq = rng.integers(-127, 128, size=(E, d)).astype(np.int8)
    Ws = (2.0 ** rng.integers(-12, -6, size=(E, d // 32))).astype(np.float32)
    Wr = (Wq.astype(np.float32) * np.repeat(Ws, 32, axis=1)).astype(np.float32)
    x = synthetic.normal(rng, 3, d)
    a = oracle.route_q8(Wq, Ws, k, x=x)
    b = oracle.route(x, Wr, k)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_route_q8_int8_equals_float_when_x_is_q8_exact():
    # x exactly the dequantised form of (xq, xs) with power-of-two scales and
    # a few nonzero words: both modes' logits are exact, so they agree bit for
    # bit, and so do the choices and weights
    rng = np.random.default_rng(66)
    E, d, k = 32, 128, 4
    Wq = rng.integers(-127, 128, size=(E, d)).astype(np.int8)
    Ws = (2.0 ** rng.integers(-10, -6, size=(E, d // 32))).astype(np.float32)
    xq = rng.integers(-127, 128, size=(2, d)).astype(np.int8)
    xs = (2.0 ** rng.integers(-9, -5, size=(2, d // 32))).astype(np.float32)
    x = (xq.astype(np.float32) * np.repeat(xs, 32, axis=1)).astype(np.float32)
    a = oracle.route_q8(Wq, Ws, k, x=x)
    b = oracle.route_q8(Wq, Ws, k, xq=xq, xs=xs)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_route_q8_two_words_brute_force_and_exact_rows():
    # two-word logits: exact rationals of sum_b ws*xs*(isum_hi + isum_lo/128);
    # brute force over the K-subsets; and on rows the two words represent
    # exactly, the same routing and logits as the float router over the rows
    rng = np.random.default_rng(95)
    E, d, k = 6, 64, 2
    Wq, Ws = _rand_q8(rng, E, d)
    x = synthetic.normal(rng, 2, d)
    xq, xl, xs = oracle.quantize_x2(x)
    idx, wts, logits = oracle.route_q8(Wq, Ws, k, xq=xq, xs=xs, xl=xl)
    for i in range(2):
        l = [sum(Fraction(float(Ws[e, b])) * Fraction(float(xs[i, b])) *
                 sum(int(Wq[e, t]) * (Fraction(int(xq[i, t])) + Fraction(int(xl[i, t]), 128))
                     for t in range(32 * b, 32 * b + 32)) for b in range(2)) for e in range(E)]
        for e in range(E):
            assert abs(Fraction(logits[i, e]) - l[e]) <= abs(l[e]) * Fraction(2) ** -50 + Fraction(2) ** -80
        best = max(itertools.combinations(range(E), k), key=lambda c: (sorted((l[j] for j in c), reverse=True), [-j for j in c]))
        assert set(idx[i]) == set(best)
    q = rng.integers(-126, 127, size=(1, d)).astype(np.int64)
    lo = rng.integers(-63, 64, size=(1, d)).astype(np.int64)
    q[:, ::32] = 127
    lo[:, ::32] = 0
    xe = ((2.0 ** -6) * (q + lo / 128.0)).astype(np.float32)
    eq, el, es = oracle.quantize_x2(xe)
    i2, w2, l2 = oracle.route_q8(Wq, Ws, k, xq=eq, xs=es, xl=el)
    i0, w0, l0 = oracle.route_q8(Wq, Ws, k, x=xe)
    assert np.array_equal(i2, i0) and np.max(np.abs(l2 - l0)) <= 1e-12 * np.max(np.abs(l0))


def test_moe_shared_two_words_with_q8_router():
    # the Q8_0 router under two words routes as route_q8 over the row's two
    # words; the shared expert's part equals its own two-word dense FFN
    v, m, x = _variant(96, sdff=128)
    idx, wts, h, y = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 2, Wrq=v.Wrq, Wrs=v.Wrs,
                                       shared=_shared(v))
    xq, xl, xs = oracle.quantize_x2(x)
    ridx, rw, _ = oracle.route_q8(v.Wrq, v.Wrs, 2, xq=xq, xs=xs, xl=xl)
    assert np.array_equal(idx, ridx) and np.array_equal(wts, rw)
    _, _, h0, y0 = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 2, Wrq=v.Wrq, Wrs=v.Wrs)
    # the shared part alone: a one-expert mixture of the shared weights
    _, _, hs1, ys1 = oracle.moe(x, np.zeros((1, x.shape[1]), np.float32), v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds,
                                1, 2)
    assert np.max(np.abs((y - y0) - ys1)) <= 1e-12 * np.max(np.abs(ys1))
    assert np.array_equal(h[:, 2 * m.Wgq.shape[0] // m.Wr.shape[0]:], hs1[:, 0])


def test_route_q8_scale_index_is_row_then_block():
    # one row of ones per expert, scale 2^-e on block e+1 (mod 4) of row e
    # and 0 elsewhere: expert e's logit is 2^-e times that block's sum of x
    # (a transposed scale index would read block e-1)
    E, d = 4, 128
    Wq = np.ones((E, d), np.int8)
    Ws = np.zeros((E, d // 32), np.float32)
    for e in range(E):
        Ws[e, (e + 1) % 4] = 2.0 ** -e
    x = np.zeros((1, d), np.float32)
    x[0, :] = np.repeat(np.array([1.0, 8.0, 64.0, 512.0], np.float32), 32)
    _, _, logits = oracle.route_q8(Wq, Ws, 1, x=x)
    assert list(logits[0]) == [256.0, 1024.0, 4096.0, 4.0]


# ---------------------------------------------------------------------------
# M: the MoE block


def _deq(q, s):
    return q.astype(np.float64) * np.repeat(s.astype(np.float64), 32, axis=1)


def _dense_swiglu(x, Wg, Wu, Wd):
    """A dense SwiGLU FFN in numpy float64, its hidden row held in float32."""
    g = Wg @ x
    u = Wu @ x
    hid = (g / (1.0 + np.exp(-g)) * u).astype(np.float32).astype(np.float64)
    return Wd @ hid, hid


def _small_moe(seed, d=64, dff=96, E=4, k=2, rows=2):
    return synthetic.moe_inputs(seed, d, dff, E, k, rows)


def test_moe_single_expert_is_dense_swiglu():
    m = _small_moe(61, E=1, k=1, rows=2)
    idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 1, act=0)
    assert (idx == 0).all() and (wts == 1.0).all()
    for i in range(2):
        ref, hid = _dense_swiglu(m.x[i].astype(np.float64), _deq(m.Wgq, m.Wgs), _deq(m.Wuq, m.Wus), _deq(m.Wdq, m.Wds))
        assert np.max(np.abs(h[i, 0] - hid)) == 0.0
        assert np.max(np.abs(y[i] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_all_experts_is_softmax_mixture():
    m = _small_moe(62, E=4, k=4, rows=3)
    idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 4, act=0)
    d, dff = m.d, m.dff
    for i in range(3):
        l = m.Wr.astype(np.float64) @ m.x[i].astype(np.float64)
        p = scipy.special.softmax(l)
        ref = np.zeros(d)
        for e in range(4):
            ye, _ = _dense_swiglu(m.x[i].astype(np.float64),
                                  _deq(m.Wgq[e * dff:(e + 1) * dff], m.Wgs[e * dff:(e + 1) * dff]),
                                  _deq(m.Wuq[e * dff:(e + 1) * dff], m.Wus[e * dff:(e + 1) * dff]),
                                  _deq(m.Wdq[e * d:(e + 1) * d], m.Wds[e * d:(e + 1) * d]))
            ref += p[e] * ye
        assert np.max(np.abs(y[i] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_identical_experts_any_router_is_dense():
    base = _small_moe(63, E=1, k=1, rows=2)
    E, d, dff = 3, base.d, base.dff
    Wr = (0.02 * synthetic.normal(np.random.default_rng(64), E, d)).astype(np.float32)
    rep = lambda a: np.concatenate([a] * E, axis=0)
    idx, wts, h, y = oracle.moe(base.x, Wr, rep(base.Wgq), rep(base.Wgs), rep(base.Wuq), rep(base.Wus),
                                rep(base.Wdq), rep(base.Wds), E, act=0)
    for i in range(2):
        ref, _ = _dense_swiglu(base.x[i].astype(np.float64), _deq(base.Wgq, base.Wgs), _deq(base.Wuq, base.Wus),
                               _deq(base.Wdq, base.Wds))
        assert np.max(np.abs(y[i] - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_int8_gate_up_exact_when_x_is_q8_exact():
    # x of integers with |x| reaching 127 in every block quantises exactly
    # (d = 1, q = x), so the int8 mode's hidden row equals the f32 mode's.
    m = _small_moe(65, E=4, k=2, rows=1)
    rng = np.random.default_rng(66)
    x = rng.integers(-126, 127, size=(1, m.d)).astype(np.float32)
    x[0, ::32] = 127.0
    _, _, hf, _ = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=0)
    _, _, hi, _ = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=1)
    assert np.max(np.abs(hi - hf) / (np.abs(hf) + 1e-30)) <= 2.0 ** -23


def test_moe_int8_within_bound_of_f32_mode():
    m = _small_moe(67, d=128, dff=128, E=4, k=2, rows=2)
    _, _, _, yf = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=0)
    _, _, _, yi = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=1)
    assert np.max(np.abs(yi - yf)) <= 3e-2 * np.max(np.abs(yf))


def test_moe_chunk_rows_are_independent():
    m = _small_moe(68, E=6, k=2, rows=5)
    for act in (0, 1, 2):
        idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=act)
        for i in range(5):
            i1, w1, h1, y1 = oracle.moe(m.x[i:i + 1], m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=act)
            assert np.array_equal(idx[i], i1[0]) and np.array_equal(y[i], y1[0]) and np.array_equal(h[i], h1[0])


def test_moe_rejects_unknown_mode():
    m = _small_moe(69, E=2, k=1, rows=1)
    with pytest.raises(AssertionError):
        oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 1, act=3)


def test_moe_x2_gate_up_exact_when_x_is_two_word_exact():
    # x the two words represent exactly (power-of-two block scales, a word of
    # 127 in every block, low words within +-63): the two-word mode's hidden
    # row equals the f32 mode's
    m = _small_moe(80, d=128, E=4, k=2, rows=1)
    rng = np.random.default_rng(81)
    q = rng.integers(-126, 127, size=(1, m.d)).astype(np.int64)
    lo = rng.integers(-63, 64, size=(1, m.d)).astype(np.int64)
    q[:, ::32] = 127
    lo[:, ::32] = 0
    dd = 2.0 ** rng.integers(-8, -4, size=(1, m.d // 32))
    x = (np.repeat(dd, 32, axis=1) * (q + lo / 128.0)).astype(np.float32)
    _, _, hf, _ = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=0)
    _, _, h2, _ = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=2)
    assert np.max(np.abs(h2 - hf) / (np.abs(hf) + 1e-30)) <= 2.0 ** -23


def test_moe_x2_within_bound_of_f32_mode_and_inside_one_word():
    m = _small_moe(82, d=128, dff=128, E=4, k=2, rows=2)
    _, _, _, yf = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=0)
    _, _, _, y1 = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=1)
    _, _, _, y2 = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=2)
    assert np.max(np.abs(y2 - yf)) <= 3e-2 / 64 * np.max(np.abs(yf))
    assert np.max(np.abs(y2 - yf)) < np.max(np.abs(y1 - yf)) / 16


def test_moe_x2_routes_as_f32():
    # the float router reads the f32 row in every numerics
    m = _small_moe(83, E=6, k=3, rows=3)
    i0, w0, _, _ = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 3, act=0)
    i2, w2, _, _ = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 3, act=2)
    assert np.array_equal(i0, i2) and np.array_equal(w0, w2)


# The down projection of the int8 numerics reads the hidden row's quantised
# form (arena.rs fn scratch: hq/hs over K*dff; qwen_emit fn moe_dp4a_kernels:
# quantize, then gate-up-SwiGLU, then down-combine).  With down rows that are
# unit vectors of power-of-two scale, every output of an expert's down
# projection is one hidden value exactly as the down kernel sees it, so the
# block's output exposes the hidden row's codes: they must be the brute-force
# nearest codes of the float32 hidden row (one word), or its brute-force words
# and low words (two words).  A down projection fed the float32 row itself, or
# the wrong word count, moves every output by a fraction of a step.


def _identity_down(m, E, scale_exp=0):
    """m's experts with down rows e_o (output o reads hidden value o) of
    scale 2**scale_exp: Wd[e*d + o, t] = (t == o), d == dff."""
    d, dff = m.d, m.dff
    assert d == dff
    Wdq = np.tile(np.eye(d, dtype=np.int8), (E, 1))
    Wds = np.full((E * d, dff // 32), 2.0 ** scale_exp, np.float32)
    return Wdq, Wds


def _block_codes(hrow):
    """Brute-force one-word codes and float32 scales of a float32 hidden row,
    from the quantiser's definition: d = amax/127 and id = 1/d in float32,
    then the nearest code to the float32 product v*id, ties away from zero."""
    hrow = np.asarray(hrow, np.float32)
    codes = np.empty(hrow.shape, np.int64)
    dsc = np.empty(hrow.shape[0] // 32, np.float32)
    for b in range(hrow.shape[0] // 32):
        blk = hrow[b * 32:(b + 1) * 32]
        dd = np.float32(np.max(np.abs(blk))) / np.float32(127.0)
        idv = np.float32(1.0) / dd if dd != 0 else np.float32(0.0)
        dsc[b] = dd
        for t in range(32):
            codes[b * 32 + t] = _nearest_away(np.float32(blk[t]) * idv)
    return codes, dsc


@pytest.mark.parametrize("seed", [90, 91])
def test_moe_int8_down_reads_brute_force_codes_of_hidden_row(seed):
    m = _small_moe(seed, d=64, dff=64, E=3, k=1, rows=2)
    Wdq, Wds = _identity_down(m, 3)
    idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, Wdq, Wds, 1, act=1)
    assert (wts == 1.0).all()
    moved = 0.0
    for i in range(2):
        codes, dsc = _block_codes(h[i, 0])
        want = np.repeat(dsc.astype(np.float64), 32) * codes
        assert np.array_equal(y[i], want), (i, np.max(np.abs(y[i] - want)))
        moved = max(moved, np.max(np.abs(want - h[i, 0].astype(np.float64))))
    # the codes are not the float row: a down projection of the row itself fails
    assert moved > 1e-6 * np.max(np.abs(h))


def test_moe_int8_down_codes_weighted_over_two_slots():
    # K = 2: y = w0 * deq(Q(h0)) + w1 * deq(Q(h1)) in double, slot order
    m = _small_moe(92, d=64, dff=64, E=4, k=2, rows=2)
    Wdq, Wds = _identity_down(m, 4, scale_exp=-1)
    idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, Wdq, Wds, 2, act=1)
    for i in range(2):
        want = np.zeros(64)
        for j in range(2):
            codes, dsc = _block_codes(h[i, j])
            want += wts[i, j] * (0.5 * np.repeat(dsc.astype(np.float64), 32) * codes)
        assert np.max(np.abs(y[i] - want)) <= 1e-15 * np.max(np.abs(want))
        assert abs(wts[i].sum() - 1.0) <= 1e-15


@pytest.mark.parametrize("seed", [93, 94])
def test_moe_x2_down_reads_brute_force_two_words_of_hidden_row(seed):
    m = _small_moe(seed, d=64, dff=64, E=3, k=1, rows=2)
    Wdq, Wds = _identity_down(m, 3)
    idx, wts, h, y = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, Wdq, Wds, 1, act=2)
    _, _, _, y1 = oracle.moe(m.x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, Wdq, Wds, 1, act=1)
    assert (wts == 1.0).all()
    for i in range(2):
        hrow = h[i, 0]
        codes, dsc = _block_codes(hrow)
        lows = np.empty(64, np.int64)
        for t in range(64):
            dd = dsc[t // 32]
            idv = np.float32(1.0) / dd if dd != 0 else np.float32(0.0)
            lows[t] = _low_word_brute_force(np.float32(hrow[t]) * idv, int(codes[t]))
        want = np.repeat(dsc.astype(np.float64), 32) * (codes * 128 + lows) / 128.0
        assert np.array_equal(y[i], want), (i, np.max(np.abs(y[i] - want)))
        # two words are not one word and not the float row
        assert not np.array_equal(y[i], y1[i])
        assert not np.array_equal(y[i], hrow.astype(np.float64))


def _discriminating_router(x, deq, E=2, seed=95):
    """Float32 router rows [E, d] whose top-1 expert differs between the row x
    and its dequantised form deq: rows 1.. add to row 0 a direction whose
    logit gap is +D/2 on x and -D/2 on deq (D = |x - deq|^2 > 0)."""
    rng = np.random.default_rng(seed)
    x = x.astype(np.float64)
    deq = deq.astype(np.float64)
    delta = x - deq
    w = rng.standard_normal(x.shape[0])
    # gap(s) on x: delta.x + s*w.x; on deq: delta.deq + s*w.deq; their
    # difference is |delta|^2 + s*w.delta; set gap on x to half of that
    D2 = float(delta @ delta)
    s = (D2 / 2 - float(delta @ x)) / (float(w @ x) - float(w @ delta) / 2)
    v = delta + s * w
    base = 0.02 * rng.standard_normal(x.shape[0])
    Wr = np.stack([base] + [base + v * (1.0 + 0.01 * e) for e in range(1, E)]).astype(np.float32)
    return Wr


@pytest.mark.parametrize("act", [1, 2])
def test_moe_int8_routes_from_float_row_not_its_quantised_form(act):
    # a float32 router reads the float32 row in the int8 numerics too (lane_link
    # fn only_projections: a reader that is not a Q8_0 projection keeps the
    # norm's float output); on this router the row and its quantised form pick
    # different experts, so a block that routed from the quantised row fails
    m = _small_moe(96, d=64, dff=64, E=2, k=1, rows=1)
    if act == 1:
        xq, xs = oracle.quantize(m.x)
        deq = xq[0].astype(np.float64) * np.repeat(xs[0].astype(np.float64), 32)
    else:
        xq, xl, xs = oracle.quantize_x2(m.x)
        deq = (xq[0].astype(np.float64) + xl[0] / 128.0) * np.repeat(xs[0].astype(np.float64), 32)
    Wr = _discriminating_router(m.x[0], deq)
    lx = Wr.astype(np.float64) @ m.x[0].astype(np.float64)
    ld = Wr.astype(np.float64) @ deq
    assert int(np.argmax(lx)) != int(np.argmax(ld)), (lx, ld)
    idx, wts, _, _ = oracle.moe(m.x, Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 1, act=act)
    assert idx[0, 0] == int(np.argmax(lx)) and wts[0, 0] == 1.0


# ---------------------------------------------------------------------------
# MS: the mixture with a shared expert and/or Q8_0 router rows


def _variant(seed, d=64, dff=96, E=4, k=2, rows=2, sdff=128):
    v = synthetic.variant_inputs(seed, d, dff, E, k, rows, sdff)
    m = v.block.moe
    x = synthetic.normal(np.random.default_rng(seed + 1000), rows, d)
    return v, m, x


def _shared(v):
    return (v.Sgq, v.Sgs, v.Suq, v.Sus, v.Sdq, v.Sds)


def test_moe_shared_without_variants_is_moe():
    v, m, x = _variant(71)
    for act in (0, 1, 2):
        a = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=act)
        b = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act, Wr=m.Wr)
        for u, w in zip(a, b):
            assert np.array_equal(u.reshape(w.shape), w)


def test_moe_shared_expert_adds_a_dense_swiglu():
    # the shared expert's part is the numpy dense SwiGLU of its own weights,
    # added with weight 1; its hidden row follows the K routed ones
    v, m, x = _variant(72, sdff=160)
    idx0, wts0, h0, y0 = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=0)
    idx, wts, h, y = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 0, Wr=m.Wr,
                                       shared=_shared(v))
    assert np.array_equal(idx, idx0) and np.array_equal(wts, wts0)
    assert np.array_equal(h[:, :2 * m.dff], h0.reshape(2, -1))
    for i in range(2):
        ref, hid = _dense_swiglu(x[i].astype(np.float64), _deq(v.Sgq, v.Sgs), _deq(v.Suq, v.Sus), _deq(v.Sdq, v.Sds))
        assert np.array_equal(h[i, 2 * m.dff:], hid.astype(np.float32))
        assert np.max(np.abs((y[i] - y0[i]) - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_moe_shared_expert_equal_to_the_only_expert_doubles_it():
    # one routed expert (weight 1) and a shared expert with the same weights:
    # the output is exactly twice the dense SwiGLU (x + x is exact)
    v, m, x = _variant(73, E=1, k=1, sdff=96)
    sh = (m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds)
    for act in (0, 1):
        _, wts, h, y = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 1, act, Wr=m.Wr, shared=sh)
        _, _, h1, y1 = oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 1, act=act)
        assert (wts == 1.0).all()
        assert np.array_equal(h[:, :96], h[:, 96:]) and np.array_equal(h[:, :96], h1.reshape(2, 96))
        assert np.array_equal(y, 2.0 * y1)


def test_moe_q8_router_routes_as_route_q8():
    v, m, x = _variant(74, E=8, k=3, rows=3, sdff=0)
    for act in (0, 1):
        idx, wts, _, _ = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 3, act,
                                           Wrq=v.Wrq, Wrs=v.Wrs)
        if act == 0:
            ri, rw, _ = oracle.route_q8(v.Wrq, v.Wrs, 3, x=x)
        else:
            xq, xs = oracle.quantize(x)
            ri, rw, _ = oracle.route_q8(v.Wrq, v.Wrs, 3, xq=xq, xs=xs)
        assert np.array_equal(idx, ri) and np.array_equal(wts, rw)


def test_moe_q8_router_on_exact_rows_equals_float_router():
    # power-of-two router scales: the Q8_0 rows' dequantised form is exact in
    # float32, so in f32 numerics the block equals the block on those rows
    v, m, x = _variant(75, E=6, k=2, rows=2, sdff=64)
    rng = np.random.default_rng(76)
    Wrs = (2.0 ** rng.integers(-12, -8, size=v.Wrs.shape)).astype(np.float32)
    Wr = (v.Wrq.astype(np.float32) * np.repeat(Wrs, 32, axis=1)).astype(np.float32)
    a = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 0, Wrq=v.Wrq, Wrs=Wrs, shared=_shared(v))
    b = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 0, Wr=Wr, shared=_shared(v))
    for u, w in zip(a, b):
        assert np.array_equal(u, w)


def test_moe_shared_int8_within_bound_of_f32_mode():
    v, m, x = _variant(77, d=128, dff=128, E=4, k=2, rows=2, sdff=256)
    _, _, _, yf = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 0, Wr=m.Wr, shared=_shared(v))
    _, _, _, yi = oracle.moe_shared(x, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, 1, Wr=m.Wr, shared=_shared(v))
    assert np.max(np.abs(yi - yf)) <= 3e-2 * np.max(np.abs(yf))


def test_oracle_refuses_non_finite_inputs():
    # NaN and infinity have no reading on the pages: the oracle refuses them
    # (the library's own NaN ranking is checked against the test's rule)
    m = _small_moe(97, E=4, k=2, rows=1)
    for bad in (np.nan, np.inf, -np.inf):
        x = m.x.copy()
        x[0, 3] = bad
        with pytest.raises(AssertionError, match="finite"):
            oracle.route(x, m.Wr, 2)
        with pytest.raises(AssertionError, match="finite"):
            oracle.moe(x, m.Wr, m.Wgq, m.Wgs, m.Wuq, m.Wus, m.Wdq, m.Wds, 2, act=1)
        with pytest.raises(AssertionError, match="finite"):
            oracle.quantize(x)
        with pytest.raises(AssertionError, match="finite"):
            oracle.gemv_f32(m.Wgq[:4], m.Wgs[:4], x)
