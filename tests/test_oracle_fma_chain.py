"""Pins of the oracle's fp32 accumulation: fma_f32 (a*b + c rounded once to
fp32) and the combines built on it (slot-order fp32 chains, one bf16
rounding at the end).

fma_f32 is checked against an independent correct rounding written with
Python Fractions: the exact value a*b + c, its binade found by comparison,
the quantum 2^(e-23) (2^-149 below the smallest normal), and rounding half
to even on the exact quotient. The inputs include random values over the
whole exponent range, subnormal products and sums, signed zeros, and the
cases where rounding the fp64 sum first and then to fp32 goes wrong (the
fp64 sum lands exactly on an fp32 midpoint while the exact sum does not).

The combines are checked against per-element chains written with the same
Fraction rounding, against a hand-worked example in which the slot order
decides the result, and against the exact sum within the chain's error
bound."""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W
from exact_f32 import chain_rows_bf16, fma_ref as _fma_ref  # noqa: E402

def _same_bits(u, v) -> bool:
    return np.float32(u).view(np.uint32) == np.float32(v).view(np.uint32)


def _random_f32(g, n, emin, emax):
    m = g.integers(0, 1 << 23, n, dtype=np.uint32)
    e = g.integers(emin + 127, emax + 127 + 1, n).astype(np.uint32)
    s = g.integers(0, 2, n, dtype=np.uint32) << 31
    return (s | (e << 23) | m).view(np.float32)


def _check_many(a, b, c):
    got = O.fma_f32(a, b, c)
    for i in range(len(a)):
        want = _fma_ref(a[i], b[i], c[i])
        assert _same_bits(got[i], want), (i, a[i], b[i], c[i], got[i], want)


def test_fma_random_wide_exponents():
    g = np.random.Generator(np.random.PCG64(7))
    n = 3000
    a = _random_f32(g, n, -45, 45)
    b = _random_f32(g, n, -45, 45)
    # c near the product's magnitude, so that cancellation and carries occur
    p = a.astype(np.float64) * b.astype(np.float64)
    c = (p * g.uniform(-2.0, 2.0, n)).astype(np.float32)
    _check_many(a, b, c)
    # c far above and far below the product
    _check_many(a, b, (p * 2.0 ** 30).astype(np.float32))
    _check_many(a, b, (p * 2.0 ** -30).astype(np.float32))


def test_fma_subnormal_products_and_sums():
    g = np.random.Generator(np.random.PCG64(8))
    n = 2000
    a = _random_f32(g, n, -75, -55)
    b = _random_f32(g, n, -75, -55)               # products 2^-150..2^-109
    c = _random_f32(g, n, -126, -110)
    sub = (g.integers(0, 1 << 23, n, dtype=np.uint32)
           | (g.integers(0, 2, n, dtype=np.uint32) << 31)).view(np.float32)
    _check_many(a, b, c)
    _check_many(a, b, sub)                          # c subnormal
    _check_many(sub, np.full(n, 1.5, np.float32), sub[::-1].copy())


def test_fma_midpoint_after_fp64_rounding():
    """a*b + c with a = +-(1 + 2^-23), b = 1 - 2^-23 (product 1 - 2^-46) and
    c = 2^24 + 2, 4 or 6: the fp64 sum is exactly an fp32 midpoint (2^24 + 1,
    3 or 5), while the exact sum lies 2^-46 to one side. Rounding the fp64
    sum to fp32 picks the even neighbour; the correct result is the
    neighbour on the side of the exact sum, which differs from the even one
    in three of the four families. Checked at many scales and both signs,
    against the Fraction reference and against the values worked out by
    hand."""
    a1 = np.float32(1 + 2.0 ** -23)
    b1 = np.float32(1 - 2.0 ** -23)
    cases = []
    for scale in range(-100, 101, 5):
        f = 2.0 ** scale
        for c0, sa, want in [(2.0 ** 24 + 2, 1, 2.0 ** 24 + 2),     # x = 2^24 + 3 - 2^-46
                             (2.0 ** 24 + 6, -1, 2.0 ** 24 + 6),    # x = 2^24 + 5 + 2^-46
                             (2.0 ** 24 + 2, -1, 2.0 ** 24 + 2),    # x = 2^24 + 1 + 2^-46
                             (2.0 ** 24 + 4, 1, 2.0 ** 24 + 4)]:    # x = 2^24 + 5 - 2^-46
            for sg in (1.0, -1.0):
                cases.append((np.float32(sg * sa * a1 * f), b1, np.float32(sg * c0 * f),
                              sg * want * f))
    a = np.array([x[0] for x in cases], np.float32)
    b = np.array([x[1] for x in cases], np.float32)
    c = np.array([x[2] for x in cases], np.float32)
    got = O.fma_f32(a, b, c)
    for i, (_, _, _, want) in enumerate(cases):
        assert float(got[i]) == want, (i, got[i], want)
        assert _same_bits(got[i], _fma_ref(a[i], b[i], c[i]))
    # the naive fp64-then-fp32 rounding differs on three of the four families
    naive = (a.astype(np.float64) * b + c).astype(np.float32)
    assert (naive != got).sum() == 3 * len(cases) // 4


def test_fma_midpoint_tail_in_addend():
    """The other side of the two-sum: a*b = (2^12 + 1)(2^12 + 3) = 2^24 + 16387,
    an fp32 midpoint, and c = +-2^-30 carries the tail below fp64 precision.
    With c = -2^-30 the result is 2^24 + 16386, with c = +2^-30 it is
    2^24 + 16388 (worked by hand; the even neighbour is 16388 either way)."""
    a1, b1 = np.float32(2.0 ** 12 + 1), np.float32(2.0 ** 12 + 3)
    a, b, c, want = [], [], [], []
    for scale in range(-60, 61, 4):
        f = 2.0 ** scale
        for sc, w in ((-1.0, 2.0 ** 24 + 16386), (1.0, 2.0 ** 24 + 16388)):
            for sg in (1.0, -1.0):
                a.append(np.float32(sg * a1 * f))
                b.append(b1)
                c.append(np.float32(sg * sc * 2.0 ** -30 * f))
                want.append(sg * w * f)
    a, b, c = (np.array(v, np.float32) for v in (a, b, c))
    got = O.fma_f32(a, b, c)
    assert np.array_equal(got.astype(np.float64), np.array(want))
    for i in range(len(a)):
        assert _same_bits(got[i], _fma_ref(a[i], b[i], c[i]))


def test_fma_signed_zeros():
    z, nz = np.float32(0.0), np.float32(-0.0)
    one = np.float32(1.0)
    rows = [(one, nz, z, z),       # -0 + +0 = +0
            (one, nz, nz, nz),     # -0 + -0 = -0
            (-one, z, nz, nz),
            (one, z, nz, z),
            (one, one, -one, z)]   # exact cancellation gives +0
    for a, b, c, want in rows:
        got = O.fma_f32(np.array([a]), np.array([b]), np.array([c]))[0]
        assert _same_bits(got, want), (a, b, c, got)
        assert _same_bits(got, _fma_ref(a, b, c))


def test_combine_equals_fraction_chain():
    g = np.random.Generator(np.random.PCG64(31))
    t, k, rows, h = 24, 6, 80, 12
    # rows with mixed magnitudes and signs, so that the chain rounds and
    # cancels
    y = W.random_bf16_rows(g, rows, h)
    big = O.round_to_bf16(O.bf16_to_f32(y).astype(np.float64) * 2.0 ** 12)
    y[::3] = big[::3]
    dst = np.stack([g.permutation(rows)[:k] for _ in range(t)]).astype(np.int32)
    dst[2, 0] = -1
    dst[5, 3:] = -1
    wt = W.random_weights(g, t, k)
    out, _ = O.combine(y, dst, wt)
    for i in range(t):
        live = [j for j in range(k) if dst[i, j] >= 0]
        want = chain_rows_bf16([wt[i, j] for j in live], [y[dst[i, j]] for j in live])
        assert np.array_equal(out[i], want), i


def test_combine_slot_order_decides_hand_example():
    """Three unit-weight slots y = 1, 1.5*2^-24, -1 (all bf16 values). In slot
    order the fp32 chain gives 1 + 1.5*2^-24 -> 1 + 2^-23 (nearest fp32),
    then 2^-23: the output is 2^-23. The exact sum is 1.5*2^-24, which the
    reversed order 1, -1, 1.5*2^-24 reaches exactly."""
    vals = np.array([1.0, 1.5 * 2.0 ** -24, -1.0])
    y = O.round_to_bf16(vals).reshape(3, 1)
    assert np.array_equal(O.bf16_to_f32(y)[:, 0], vals.astype(np.float32))
    w = np.ones((1, 3), np.float32)
    out, _ = O.combine(y, np.array([[0, 1, 2]], np.int32), w)
    assert float(O.bf16_to_f32(out)[0, 0]) == 2.0 ** -23
    rev, _ = O.combine(y, np.array([[0, 2, 1]], np.int32), w)
    assert float(O.bf16_to_f32(rev)[0, 0]) == 1.5 * 2.0 ** -24
    # the gradient of dispatch is the same unit-weight chain
    dx, _ = O.dispatch_backward(y, np.array([[0, 1, 2]], np.int32))
    assert np.array_equal(dx, out)


def test_combine_midpoint_through_bf16_inputs():
    """A combine whose second step lands the fp64 sum on an fp32 midpoint:
    y = 2^24, 1.015625, -2^24 (bf16) with w = 1 + 2^-22, w1, 1 where
    w1 = 0.98461538553... is the fp32 value with w1 * 1.015625 = 1 + 2^-30.
    Step 1 gives 2^24 + 4; step 2 the exact 2^24 + 5 + 2^-30, which rounds up
    to 2^24 + 6; step 3 leaves 6. Rounding through fp64 would give 4, and
    the exact sum 5 + 2^-30 rounds to 5 in bf16."""
    w1 = np.float32(0.9846153855323792)
    assert Fraction(float(w1)) * Fraction(65, 64) == 1 + Fraction(1, 2 ** 30)
    y = O.round_to_bf16(np.array([2.0 ** 24, 1.015625, -(2.0 ** 24)])).reshape(3, 1)
    w = np.array([[1 + 2.0 ** -22, w1, 1.0]], np.float32)
    out, _ = O.combine(y, np.array([[0, 1, 2]], np.int32), w)
    assert float(O.bf16_to_f32(out)[0, 0]) == 6.0


def test_combine_local_and_partials_are_slot_order_chains():
    """Rank rows with several slots: each partial is the fp32 chain of its
    slots in slot order; the partial sum is the unit-weight chain of the
    partials in slot order of the ranks' first slots. The slots 1, -1,
    1.5*2^-24 sum exactly in slot order; reversed they would give 2^-23
    (-1 + 1.5*2^-24 is an fp32 tie that goes to -1 + 2^-23)."""
    vals = np.array([1.0, -1.0, 1.5 * 2.0 ** -24, 2.0 ** -22])
    y = O.round_to_bf16(vals).reshape(4, 1)
    dst = np.array([[0, 1, 2, 3]], np.int32)
    w = np.ones((1, 4), np.float32)
    rank_row = np.array([[0, 0, 0, 1]], np.int32)   # slots 0..2 on one rank
    part, written, _ = O.combine_local(y, dst, rank_row, w, 2)
    assert written.all()
    assert float(O.bf16_to_f32(part)[0, 0]) == 1.5 * 2.0 ** -24
    assert float(O.bf16_to_f32(part)[1, 0]) == 2.0 ** -22
    send_row = np.array([[0, -1, -1, 1]], np.int32)
    out, _ = O.combine_partials(part, send_row)
    assert float(O.bf16_to_f32(out)[0, 0]) == 1.375 * 2.0 ** -22


@pytest.mark.parametrize("seed", [0, 1])
def test_combine_chain_within_bound_of_exact_sum(seed):
    """The chain's error against the exact sum: at most half a bf16 ulp of
    output plus n * 2^-24 * sum|w y| for n live slots (each of the n fp32
    steps rounds once, with relative error at most 2^-24 of a partial sum)."""
    g = np.random.Generator(np.random.PCG64(40 + seed))
    t, k, rows, h = 30, 8, 200, 16
    y = W.random_bf16_rows(g, rows, h)
    dst = np.stack([g.permutation(rows)[:k] for _ in range(t)]).astype(np.int32)
    wt = W.random_weights(g, t, k)
    out, mag = O.combine(y, dst, wt)
    yf = O.bf16_to_f32(y)
    for i in range(t):
        for c in range(h):
            terms = [float(wt[i, j]) * float(yf[dst[i, j], c]) for j in range(k)]
            exact = math.fsum(terms)
            got = float(O.bf16_to_f32(out[i:i + 1, c:c + 1])[0, 0])
            ulp = 2.0 ** (math.floor(math.log2(max(abs(got), abs(exact), 2.0 ** -126))) - 7)
            bound = ulp / 2 + k * 2.0 ** -24 * mag[i, c]
            assert abs(got - exact) <= bound * (1 + 1e-12)
