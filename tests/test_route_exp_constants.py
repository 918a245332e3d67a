"""CPU pins of the fp64 exp that the routing kernels use (route.hip:
exp_f64, sigmoid_f32). The constants are read from the kernel source itself
and checked against the mathematics they stand for; the method (Cody and
Waite's range reduction, the degree-13 Taylor series by Horner's rule, a
reciprocal refined by two Newton steps) is then run with exact fused
multiply-adds and checked against math.exp and against the oracle's fp32
sigmoid. The GPU route parity tests check the kernel itself."""

import math
import os
import re
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

from oracle import moe_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "combine_moe_layout_06_amd", "csrc", "route.hip")


def _constants():
    text = open(SRC).read()
    table = re.search(r"route_exp_taylor\[14\]\s*=\s*\{(.*?)\};", text, re.S).group(1)
    table = re.sub(r"//[^\n]*", "", table)
    coef = [float.fromhex(t.strip()) for t in table.split(",") if t.strip()]
    named = {n: float.fromhex(re.search(r"constexpr double %s = ([-0-9a-fx.p+]+);" % n,
                                        text).group(1))
             for n in ("kLog2e", "kLn2Hi", "kLn2Lo")}
    return coef, named


def _ln2():
    getcontext().prec = 80
    return Fraction(Decimal(2).ln())


def test_taylor_coefficients_are_the_nearest_doubles_of_one_over_j_factorial():
    coef, _ = _constants()
    assert len(coef) == 14
    for i, c in enumerate(coef):
        j = 13 - i
        assert c == float(Fraction(1, math.factorial(j))), j


def test_ln2_split_and_log2e():
    _, k = _constants()
    ln2 = _ln2()
    hi, lo = Fraction(k["kLn2Hi"]), Fraction(k["kLn2Lo"])
    # head: 32 significant bits, so n * head is exact for |n| < 2^21
    assert (hi * 2 ** 32).denominator == 1
    assert abs(hi - ln2) <= Fraction(1, 2 ** 33)
    assert k["kLn2Lo"] == float(ln2 - hi)
    assert abs(hi + lo - ln2) < Fraction(1, 2 ** 85)
    assert k["kLog2e"] == float(1 / ln2)


def _fma(a, b, c):
    return float(Fraction(a) * Fraction(b) + Fraction(c))


def _exp_model(x, coef, k):
    x = min(max(x, -800.0), 700.0)
    n = float(round(x * k["kLog2e"]))
    r = _fma(-n, k["kLn2Hi"], x)
    r = _fma(-n, k["kLn2Lo"], r)
    p = coef[0]
    for c in coef[1:]:
        p = _fma(p, r, c)
    return math.ldexp(p, int(n))


def _rcp_estimate(d):
    """A 24-bit reciprocal, coarser than the hardware estimate."""
    f = Fraction(1) / Fraction(d)
    e = math.frexp(float(f))[1]
    return float(Fraction(round(f * 2 ** (24 - e)), 2 ** (24 - e)))


def _sigmoid_model(lv, coef, k):
    d = 1.0 + _exp_model(-float(lv), coef, k)
    y = _rcp_estimate(d)
    y = _fma(y, _fma(-d, y, 1.0), y)
    y = _fma(y, _fma(-d, y, 1.0), y)
    return np.float32(y)


def test_exp_method_within_one_ulp():
    coef, k = _constants()
    g = np.random.default_rng(11)
    xs = np.concatenate([g.normal(0, 3, 600), g.uniform(-740, 700, 600),
                         [0.0, -0.0, 1e-300, -1e-300, 0.5 * math.log(2), -0.5 * math.log(2)]])
    for x in xs:
        ref = math.exp(x)
        if ref < 2.3e-308:          # subnormal results: not used by the sigmoid
            continue
        assert abs(_exp_model(float(x), coef, k) - ref) <= math.ulp(ref), x


def test_sigmoid_method_matches_the_oracle():
    coef, k = _constants()
    g = np.random.default_rng(12)
    ls = np.concatenate([(g.standard_normal(3000) * 4).astype(np.float32),
                         np.array([0, -0.0, 1e-30, -1e-30, 88, -88, 104, -104, 700, -700,
                                   3e38, -3e38], np.float32)])
    with np.errstate(over="ignore"):
        ref = O._sigmoid_f32(ls[None, :])[0]
    got = np.array([_sigmoid_model(v, coef, k) for v in ls], np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
