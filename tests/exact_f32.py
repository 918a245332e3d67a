"""Exact fp32 arithmetic for the oracle's pins, written with Python
Fractions: the correctly rounded fp32 value of a rational number, a fused
multiply-add (a*b + c rounded once), and a slot-order fp32 chain of
weighted bf16 values. Independent of the oracle's numpy implementation,
which uses fp64 two-sums; used only to check it."""

import math
from fractions import Fraction

import numpy as np

from oracle import moe_oracle as O

F32_MAX = Fraction(2) ** 127 * (2 - Fraction(2) ** -23)


def rn_f32(x: Fraction) -> np.float32:
    """Nearest fp32 to the exact rational x, ties to even mantissa."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = 0
    while a >= Fraction(2) ** (e + 1):
        e += 1
    while a < Fraction(2) ** e:
        e -= 1
    q = Fraction(2) ** (max(e, -126) - 23)
    n = a / q
    f = n.numerator // n.denominator
    rem = n - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    r = f * q
    if r > F32_MAX:
        return np.float32(sign * np.inf)
    return np.float32(sign * float(r))


def exact(v) -> Fraction:
    return Fraction(float(v))


def fma_ref(a, b, c) -> np.float32:
    x = exact(a) * exact(b) + exact(c)
    if x == 0:
        # an exact zero sum is +0 under round-to-nearest, unless both the
        # product and c are zeros of negative sign
        p_neg = (math.copysign(1.0, float(a)) * math.copysign(1.0, float(b))) < 0
        if float(a) * float(b) == 0 and float(c) == 0 and p_neg and math.copysign(1.0, float(c)) < 0:
            return np.float32(-0.0)
        return np.float32(0.0)
    return rn_f32(x)



def chain_f32(weights, values) -> np.float32:
    """acc = +0; acc = fma_ref(w, v, acc) for each (w, v) in order."""
    acc = np.float32(0.0)
    for wv, v in zip(weights, values):
        acc = fma_ref(np.float32(wv), np.float32(v), acc)
    return acc


def chain_rows_bf16(weights, rows):
    """Per-element slot-order chain over bf16 rows (uint16 bit arrays of
    equal length), rounded to bf16 bits at the end."""
    if not rows:
        return None
    vals = [O.bf16_to_f32(r) for r in rows]
    out = [chain_f32(weights, [v[c] for v in vals]) for c in range(len(rows[0]))]
    return O.round_to_bf16(np.array(out, np.float32))
