"""Pins of the oracle's number formats: bf16 and OCP e4m3fn.

Each codec is checked against a method that does not share its arithmetic:
brute-force nearest-value search over every code, integer round-half-even on
fp32 bit patterns, and closed forms of the formats' landmark values."""

import numpy as np
import pytest

from oracle import moe_oracle as O


# --------------------------------------------------------------------- e4m3

def test_e4m3_landmarks():
    t = O.e4m3_decode_table()
    assert t[0x7E] == 448.0                  # largest finite
    assert t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6              # smallest normal
    assert t[0x07] == 7 * 2.0 ** -9          # largest subnormal
    assert t[0x01] == 2.0 ** -9              # smallest subnormal
    assert t[0x38] == 1.0                    # exponent field 7 = bias
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t).sum() == 254       # no infinities, two NaNs
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)          # codes 0..0x7E increase
    assert np.array_equal(t[0x80:0xFF], -t[:0x7F])


def _e4m3_brute(v):
    """Nearest finite e4m3 value by exhaustive search over the 127 positive
    codes, ties to the even code, saturation by clamping the magnitude."""
    t = O.e4m3_decode_table()[:0x7F]
    a = np.minimum(np.abs(v.astype(np.float64)), 448.0)
    d = np.abs(a[:, None] - t[None, :])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one (at most two candidates)
    codes = np.arange(0x7F)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    sign = np.where(np.signbit(v), 0x80, 0).astype(np.uint8)
    return pick.astype(np.uint8) | sign


def test_e4m3_encode_all_bf16_patterns_times_scales():
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    for mult in [1.0, 0.5, 3.0, 448.0 / 3.1640625, 123.456, 2.0 ** -5, 1e4]:
        with np.errstate(over="ignore"):       # products past fp32 are dropped next
            x = (v * np.float32(mult)).astype(np.float32)
        x = x[np.isfinite(x)]
        for chunk in np.array_split(x, 16):
            assert np.array_equal(O.e4m3_encode(chunk), _e4m3_brute(chunk))


def test_e4m3_encode_exact_midpoints_round_to_even():
    t = O.e4m3_decode_table()[:0x7F]
    mid = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (t[:-1] + t[1:]) / 2)
    got = O.e4m3_encode(mid)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want.astype(np.uint8))
    # negative midpoints mirror the positive ones
    assert np.array_equal(O.e4m3_encode(-mid), want.astype(np.uint8) | 0x80)


def test_e4m3_saturation_and_signed_zero():
    v = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e30, -1e30, 0.0, -0.0,
                  2.0 ** -10, 2.0 ** -10 * 1.0001, 3 * 2.0 ** -10],
                 dtype=np.float32)
    got = O.e4m3_encode(v).tolist()
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80,
                   0x00, 0x01, 0x02]


# --------------------------------------------------------------------- bf16

def _bf16_int_rne(f32):
    """fp32 -> bf16 by integer round-half-even on the bit pattern."""
    b = f32.view(np.uint32).astype(np.uint64)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def test_round_to_bf16_matches_integer_rne_on_fp32():
    g = np.random.Generator(np.random.PCG64(7))
    b = g.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    # force many exact ties and near-ties in the low half
    b[: 1 << 16] = (b[: 1 << 16] & 0xFFFF0000) | 0x8000
    b[1 << 16: 1 << 17] = (b[1 << 16: 1 << 17] & 0xFFFF0000) | 0x7FFF
    f = b.view(np.float32)
    keep = np.isfinite(f) & (np.abs(f) < np.float32(3.38e38))
    f = f[keep]
    assert np.array_equal(O.round_to_bf16(f), _bf16_int_rne(f))


def test_round_to_bf16_fp64_is_nearest():
    """fp64 inputs (which fp32 cannot hold) round to the nearer bf16
    neighbour: compare against both neighbours of the truncated value."""
    g = np.random.Generator(np.random.PCG64(11))
    v = g.standard_normal(200000) * np.exp(g.uniform(-30, 30, 200000))
    got = O.round_to_bf16(v)
    gv = O.bf16_to_f32(got).astype(np.float64)
    lo_bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    cand = []
    for d in (-1, 0, 1):
        cb = (lo_bits.astype(np.int64) + d).astype(np.uint16)
        cand.append(O.bf16_to_f32(cb).astype(np.float64))
    cand = np.stack(cand, axis=1)
    dist = np.abs(cand - v[:, None]).min(axis=1)
    assert np.all(np.abs(gv - v) <= dist)


def test_bf16_roundtrip_identity():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    fin = np.isfinite(f)
    assert np.array_equal(O.round_to_bf16(f[fin]), bits[fin])
    assert O.bf16_to_f32(np.array([0x3F80], np.uint16))[0] == 1.0
    assert O.bf16_to_f32(np.array([0x4040], np.uint16))[0] == 3.0


@pytest.mark.parametrize("v,bits", [(1.0 + 2 ** -8, 0x3F80),            # tie -> even
                                    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie -> even
                                    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),  # past tie
                                    (2.0 ** -133, 0x0001),              # min subnormal
                                    (2.0 ** -134, 0x0000),              # tie -> 0
                                    (-0.0, 0x8000)])
def test_round_to_bf16_cases(v, bits):
    assert int(O.round_to_bf16(np.array([v]))[0]) == bits
