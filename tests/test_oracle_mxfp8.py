"""Pins of the oracle's MXFP8 quantisation (1x32 blocks, E8M0 scales):
the shared exponent is the smallest power of two that brings the block
maximum below 512, every code is the nearest e4m3 value of x / 2^e
(exhaustive search), exactly representable blocks round-trip, and the
payload plus scales take 33/64 of the bf16 bytes."""

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W


def test_exponent_brackets_the_block_maximum():
    g = np.random.Generator(np.random.PCG64(1))
    x = W.random_bf16_rows(g, 64, 512)
    x[:, 5] = (x[:, 5].astype(np.uint32) ^ 0x3000).astype(np.uint16)   # spread the exponents
    e = O.mxfp8_block_exponents(x)
    a = np.abs(O.bf16_to_f32(x).astype(np.float64)).reshape(64, 16, 32).max(axis=2)
    # 2^(e+8) <= amax < 2^(e+9), by exact comparisons
    assert np.all(np.ldexp(1.0, e + 8) <= a) and np.all(a < np.ldexp(1.0, e + 9))


def test_codes_by_exhaustive_nearest_search():
    g = np.random.Generator(np.random.PCG64(2))
    x = W.random_bf16_rows(g, 40, 256)
    codes, sb = O.quantize_mxfp8_blocks(x)
    e = sb.astype(np.int64) - 127
    v = np.ldexp(O.bf16_to_f32(x).astype(np.float64).reshape(40, 8, 32), -e[:, :, None]).reshape(-1)
    table = O.e4m3_decode_table()[:0x7F]
    d = np.abs(np.minimum(np.abs(v), 448.0)[:, None] - table[None, :])
    mag = codes.reshape(-1) & 0x7F
    assert np.all(np.abs(table[mag] - np.minimum(np.abs(v), 448.0)) == d.min(axis=1))
    assert np.all((codes.reshape(-1) >> 7) == np.signbit(v))
    # the block maximum lands in the top binade (256 .. 448)
    top = np.abs(v).reshape(40, 8, 32).argmax(axis=2)
    tc = np.take_along_axis(codes.reshape(40, 8, 32) & 0x7F, top[:, :, None], axis=2)
    assert np.all((tc >= 0x78) & (tc <= 0x7E))


def test_representable_blocks_round_trip():
    g = np.random.Generator(np.random.PCG64(3))
    table = O.e4m3_decode_table()[:0x7F]
    t = 16
    vals = table[g.integers(0x08, 0x7F, size=(t, 64))] * np.where(g.random((t, 64)) < 0.5, -1, 1)
    vals[:, ::32] = 448.0                       # each block reaches 448 = 1.75 * 2^8
    e = g.integers(-20, 20, size=(t, 2))
    x = np.ldexp(vals.reshape(t, 2, 32), e[:, :, None]).reshape(t, 64)
    bits = O.round_to_bf16(x)
    assert np.array_equal(O.bf16_to_f32(bits).astype(np.float64), x)   # exactly representable
    codes, sb = O.quantize_mxfp8_blocks(bits)
    assert np.array_equal(sb.astype(np.int64) - 127, e)
    assert np.array_equal(O.expert_dequant_mx(codes, sb), bits)


def test_zero_tiny_and_saturating_blocks():
    x = np.zeros((1, 128), dtype=np.uint16)
    x[0, 32:64] = 0x8000                         # -0 block
    x[0, 64] = 0x0001                            # smallest bf16 subnormal: exponent clamps to -127
    x[0, 96] = 0x43FF                            # 510 -> saturates to 448 (scale 2^0)
    x[0, 97] = 0x4380                            # 256 -> exact
    codes, sb = O.quantize_mxfp8_blocks(x)
    assert sb.tolist() == [[0, 0, 0, 127]]
    assert np.all(codes[0, :32] == 0) and np.all(codes[0, 32:64] == 0x80)
    assert codes[0, 64] == 0x08                 # 2^-133 / 2^-127 = 2^-6, the smallest normal
    assert codes[0, 96] == 0x7E and codes[0, 97] == 0x78


def test_payload_bytes_and_copies():
    w = W.WORKLOADS["dsv3"]
    inp = W.make_inputs(w, 4, tokens=64)
    idx, wt = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    L = O.layout(idx, w.experts, w.ranks, 0)
    q, sb, written = O.dispatch_mxfp8(inp.x, L["dst_row"], L["num_rows"])
    t, h = inp.x.shape
    assert written.all()
    assert (q.nbytes + sb.nbytes) * 64 == t * w.top_k * h * 2 * 33
    for i in range(t):
        rows = L["dst_row"][i]
        assert np.all(q[rows] == q[rows[0]]) and np.all(sb[rows] == sb[rows[0]])
    # dequantisation error: relative 2^-4 below the top code, saturation above
    codes, s1 = O.quantize_mxfp8_blocks(inp.x)
    y = O.bf16_to_f32(O.expert_dequant_mx(codes, s1)).astype(np.float64)
    xf = O.bf16_to_f32(inp.x).astype(np.float64)
    scale = np.repeat(np.ldexp(1.0, s1.astype(np.int64) - 127), 32, axis=1)
    bound = np.abs(xf) * (2.0 ** -4 + 2.0 ** -8) + scale * 2.0 ** -9 + np.maximum(np.abs(xf) - 448 * scale, 0)
    assert np.all(np.abs(y - xf) <= bound)
