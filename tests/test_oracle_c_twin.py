"""Pins of the oracle's C twin (oracle/oracle_c.c) against the numpy oracle
and against exact arithmetic (CPU only).

The twin is used where the numpy oracle is too slow (full-size parity
samples, every step of the decode sequence), so it must give the numpy
oracle's bits everywhere:
  * FP8 block quantisation: every finite bf16 pattern, placed in blocks
    under a range of block maxima (normal, subnormal and overflowing
    multipliers), plus all-zero and signed-zero blocks;
  * combine: random chains with drops, cancellation, zero and negative-zero
    terms and out-of-range rows, against moe_oracle.combine, and small
    chains against the Fraction-based fp32 chain of tests/exact_f32.py."""

import numpy as np
import pytest

from oracle import c_twin as C
from oracle import moe_oracle as O
from synth import workloads as W
from exact_f32 import chain_rows_bf16


def _finite_bf16_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = O.bf16_to_f32(bits)
    return bits[np.isfinite(v)]


def _blocks_under(maxbits, pats):
    """Rows of 128 bf16 patterns whose block maximum is |maxbits|: the first
    element is maxbits, the rest are the patterns of magnitude <= it."""
    amax = abs(float(O.bf16_to_f32(np.array([maxbits], np.uint16))[0]))
    v = np.abs(O.bf16_to_f32(pats).astype(np.float64))
    keep = pats[v <= amax]
    n = -(-len(keep) // 127)
    fill = np.resize(keep, n * 127).reshape(n, 127)
    return np.concatenate([np.full((n, 1), maxbits, np.uint16), fill], axis=1)


@pytest.mark.parametrize("maxbits", [
    0x3F80,   # 1.0
    0x4040,   # 3.0
    0x43E0,   # 448
    0x4B00,   # 2^23
    0x7F7F,   # largest finite bf16
    0x0080,   # smallest normal
    0x0001,   # smallest subnormal: 448 / amax overflows fp32
    0x0005,
    0x3A83,   # an odd mantissa
    0xC2F7,   # negative maximum
])
def test_fp8_quantise_matches_numpy_on_every_pattern(maxbits):
    x = _blocks_under(maxbits, _finite_bf16_patterns())
    # several blocks per token: 4 blocks of 128 columns
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 128), np.uint16)]).reshape(-1, 512)
    q_c, s_c = C.quantize_fp8_blocks(x)
    q_n, s_n = O.quantize_fp8_blocks(x)
    assert np.array_equal(q_c, q_n)
    assert np.array_equal(s_c.view(np.uint32), s_n.view(np.uint32))


def test_fp8_quantise_zero_blocks_and_workload_rows():
    x = np.zeros((3, 256), np.uint16)
    x[1, :128] = 0x8000                     # -0 everywhere in one block
    x[2, 5] = 0x3F80
    q_c, s_c = C.quantize_fp8_blocks(x)
    q_n, s_n = O.quantize_fp8_blocks(x)
    assert np.array_equal(q_c, q_n) and np.array_equal(s_c, s_n)
    assert np.all(q_c[1, :128] == 0x80) and s_c[1, 0] == 0.0
    inp = W.make_inputs(W.WORKLOADS["dsv3"], 5, tokens=64)
    q_c, s_c = C.quantize_fp8_blocks(inp.x)
    q_n, s_n = O.quantize_fp8_blocks(inp.x)
    assert np.array_equal(q_c, q_n)
    assert np.array_equal(s_c.view(np.uint32), s_n.view(np.uint32))


@pytest.mark.parametrize("t,h,k,rows,drop", [
    (300, 256, 8, 2400, 0.1), (200, 64, 2, 50, 0.0), (64, 128, 32, 500, 0.3),
    (0, 64, 4, 10, 0.0)])
def test_combine_matches_numpy(t, h, k, rows, drop):
    g = W.rng(t + 7 * k)
    y = W.random_bf16_rows(g, rows, h)
    y[::7, ::3] = 0x8000                      # negative zeros
    y[1::11, ::5] = 0x0000
    dst = g.integers(0, rows, size=(t, k)).astype(np.int32)
    dst[g.random((t, k)) < drop] = -1
    dst[::13, 0] = rows + 5                   # past num_rows: adds nothing
    w = W.random_weights(g, t, k)
    w[::5, 1 % k] = -w[::5, 1 % k]            # cancellation between slots
    w[::17, 0] = 0.0
    want, _ = O.combine(y, np.where(dst < rows, dst, -1).astype(np.int32), w)
    assert np.array_equal(C.combine(y, dst, w), want)
    # unit weights: the gradient of dispatch
    want1, _ = O.dispatch_backward(y, np.where(dst < rows, dst, -1).astype(np.int32))
    assert np.array_equal(C.combine(y, dst, None), want1)


def test_combine_cancellation_chains_match_numpy():
    """Large terms that cancel leave a small sum whose bits depend on every
    fp32 rounding of the chain."""
    g = W.rng(99)
    t, h, k = 400, 64, 8
    base = W.random_bf16_rows(g, t, h)
    y = np.concatenate([base, base ^ np.uint16(0x8000), W.random_bf16_rows(g, t, h)])
    dst = np.stack([np.arange(t), np.arange(t) + t] + [2 * t + np.arange(t)] * (k - 2),
                   axis=1).astype(np.int32)
    w = np.ones((t, k), np.float32)
    w[:, 1] = np.float32(1.0) + np.float32(2.0 ** -20)
    w[:, 2:] = W.random_weights(g, t, k - 2) * np.float32(2.0 ** -12)
    want, _ = O.combine(y, dst, w)
    assert np.array_equal(C.combine(y, dst, w), want)


def test_combine_matches_exact_fraction_chains():
    g = W.rng(123)
    t, h, k, rows = 12, 16, 5, 40
    y = W.random_bf16_rows(g, rows, h)
    dst = g.integers(0, rows, size=(t, k)).astype(np.int32)
    dst[2, 1] = -1
    w = (W.random_weights(g, t, k) - np.float32(0.5)).astype(np.float32)
    got = C.combine(y, dst, w)
    for i in range(t):
        live = [j for j in range(k) if dst[i, j] >= 0]
        want = chain_rows_bf16([w[i, j] for j in live], [y[dst[i, j]] for j in live])
        assert np.array_equal(got[i], want), i
