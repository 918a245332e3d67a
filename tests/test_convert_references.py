"""The integer rounding references of tests/hip/convert_sweep.hip (which
check the hardware converts on the device) checked on the host against the
oracle's codecs: every finite bf16 pattern times a range of multipliers for
e4m3, e4m3 midpoints, saturation, subnormals and zeros, and random fp32
patterns over the whole exponent range for both formats (CPU only)."""

import ctypes
import os

import numpy as np
import pytest

from oracle import moe_oracle as O

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hip", "libconvert_sweep.so")


@pytest.fixture(scope="module")
def refs():
    if not os.path.exists(LIB):
        pytest.fail("tests/hip/libconvert_sweep.so is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    for f in (lib.convert_ref_bf16, lib.convert_ref_e4m3):
        f.argtypes = [ctypes.c_uint32]
        f.restype = ctypes.c_uint32
    return lib


def _e4m3(lib, v):
    return np.array([lib.convert_ref_e4m3(int(u)) for u in v.view(np.uint32)], np.uint8)


def test_e4m3_reference_on_scaled_bf16_patterns(refs):
    bits = np.arange(1 << 16, dtype=np.uint32)
    v = (bits << 16).view(np.float32)
    v = v[np.isfinite(v)]
    g = np.random.Generator(np.random.PCG64(3))
    for mult in [1.0, 448.0 / 3.1640625, 2.0 ** -5, 1e4]:
        with np.errstate(over="ignore"):
            x = (v * np.float32(mult)).astype(np.float32)
        x = x[np.isfinite(x)]
        x = x[g.random(len(x)) < 0.25]          # a quarter of each set keeps the test short
        assert np.array_equal(_e4m3(refs, x), O.e4m3_encode(x))


def test_e4m3_reference_landmarks(refs):
    t = O.e4m3_decode_table()[:0x7F]
    mid = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    special = np.array([0.0, -0.0, 448.0, 449.0, 463.9, 464.0, 464.1, 479.0, 480.0, 1e38,
                        np.inf, -np.inf, 2.0 ** -9, 2.0 ** -10, 2.0 ** -10 * 1.0001,
                        3 * 2.0 ** -10, 2.0 ** -6, 2.0 ** -6 * (1 - 2.0 ** -5), 1e-40,
                        -1e-40], np.float32)
    x = np.concatenate([mid, -mid, t.astype(np.float32), special])
    assert np.array_equal(_e4m3(refs, x), O.e4m3_encode(np.where(np.isinf(x), np.sign(x) * 1e30, x).astype(np.float32)))


def test_both_references_on_random_fp32_patterns(refs):
    g = np.random.Generator(np.random.PCG64(4))
    u = g.integers(0, 1 << 32, 60000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    fin = np.isfinite(x)
    assert np.array_equal(_e4m3(refs, x[fin]), O.e4m3_encode(x[fin]))
    got = np.array([refs.convert_ref_bf16(int(b)) for b in u[fin]], np.uint16)
    assert np.array_equal(got, O.round_to_bf16(x[fin]))
    # infinities stay infinities, and the largest values carry into them
    for b in (0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF):
        want = O.round_to_bf16(np.array([b], np.uint32).view(np.float32))[0]
        assert refs.convert_ref_bf16(b) == want
