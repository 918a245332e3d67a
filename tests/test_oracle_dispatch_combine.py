"""Pins of the oracle's dispatch and combine: the round trip with identity
experts and normalised weights returns x exactly, FP8 payloads are half the
bf16 bytes and dequantise within the e4m3 error bound, and combine (an fp32
chain in slot order) stays within its rounding bound of an exactly summed
(math.fsum) reference on small inputs."""

import math

import numpy as np
import pytest

from oracle import moe_oracle as O
from synth import workloads as W


def _route_and_layout(w, seed, tokens):
    inp = W.make_inputs(w, seed, tokens=tokens)
    idx, wt = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    L = O.layout(idx, w.experts, w.ranks, w.capacity)
    return inp, idx, wt, L


@pytest.mark.parametrize("name", ["tiny", "mixtral", "qwen3_skew"])
def test_bf16_round_trip_identity_experts(name):
    w = W.WORKLOADS[name]
    inp, idx, wt, L = _route_and_layout(w, 0, min(w.tokens, 256))
    inp.x[3, :5] = 0x8000                   # signed zeros
    out, written = O.dispatch_bf16(inp.x, L["dst_row"], L["num_rows"])
    assert written.all()
    t = inp.x.shape[0]
    for i in range(t):
        for j in range(w.top_k):
            assert np.array_equal(out[L["dst_row"][i, j]], inp.x[i])
    back, _ = O.combine(out, L["dst_row"], wt)
    # weights sum to 1 within k fp32 ulps, far below half a bf16 ulp; compared
    # as values because a sum that starts at +0 maps an input of -0 to +0
    assert np.array_equal(O.bf16_to_f32(back), O.bf16_to_f32(inp.x))
    neg0 = inp.x == 0x8000
    assert np.all(back[neg0] == 0x0000)


def test_fp8_round_trip_and_bounds():
    w = W.WORKLOADS["dsv3"]
    inp, idx, wt, L = _route_and_layout(w, 1, 128)
    q, s, written = O.dispatch_fp8(inp.x, L["dst_row"], L["num_rows"])
    t, h = inp.x.shape
    assert written.all()
    assert q.nbytes * 2 == t * w.top_k * h * 2            # half the bf16 payload
    assert s.shape == (t * w.top_k, h // 128)
    for i in range(t):                                      # k identical copies
        rows = L["dst_row"][i]
        assert np.all(q[rows] == q[rows[0]]) and np.all(s[rows] == s[rows[0]])
    xf = O.bf16_to_f32(inp.x).astype(np.float64)
    codes, sc = O.quantize_fp8_blocks(inp.x)
    dq = O.e4m3_decode(codes).reshape(t, h // 128, 128) * sc[:, :, None].astype(np.float64)
    dq = dq.reshape(t, h)
    err = np.abs(dq - xf)
    bound = np.abs(xf) * (2.0 ** -4 + 2.0 ** -20) + np.repeat(sc, 128, axis=1) * 2.0 ** -10
    assert np.all(err <= bound)
    # the block maximum always lands on the largest code, 448
    a = np.abs(xf).reshape(t, h // 128, 128)
    m = a.argmax(axis=2)
    top = np.take_along_axis(codes.reshape(t, h // 128, 128), m[:, :, None], axis=2)
    assert np.all((top[:, :, 0] & 0x7F) == 0x7E)
    assert np.array_equal(sc, (a.max(axis=2).astype(np.float32) / np.float32(448)))
    # identity expert on the dequantised rows: combine returns bf16(q*scale)
    y = O.expert_dequant(q, s)
    back, _ = O.combine(y, L["dst_row"], wt)
    want = O.round_to_bf16((O.e4m3_decode(codes).reshape(t, -1, 128).astype(np.float32)
                            * sc[:, :, None]).astype(np.float32).reshape(t, h))
    assert np.array_equal(back, want)


def test_fp8_zero_and_tiny_blocks():
    x = np.zeros((2, 256), dtype=np.uint16)
    x[0, 128:] = 0x8000                     # -0.0
    x[1, :128] = 0x0001                     # smallest bf16 subnormal
    x[1, 5] = 0x8001
    codes, sc = O.quantize_fp8_blocks(x)
    assert np.all(codes[0, :128] == 0x00) and np.all(codes[0, 128:] == 0x80)
    assert np.all(sc[0] == 0)
    # 448/amax overflows fp32: nonzero values saturate, zeros stay zero
    assert np.all(codes[1, :128][np.arange(128) != 5] == 0x7E) and codes[1, 5] == 0xFE
    assert np.all(codes[1, 128:] == 0) and sc[1, 1] == 0 and sc[1, 0] > 0


def test_combine_within_chain_bound_of_exact_sum():
    g = np.random.Generator(np.random.PCG64(21))
    t, k, rows, h = 40, 3, 90, 16
    y = W.random_bf16_rows(g, rows, h)
    dst = np.stack([g.permutation(rows)[:k] for _ in range(t)]).astype(np.int32)
    dst[3, 1] = -1                          # a dropped pair adds nothing
    wt = W.random_weights(g, t, k)
    out, mag = O.combine(y, dst, wt)
    yf = O.bf16_to_f32(y)
    for i in range(t):
        for c in range(h):
            terms = [float(wt[i, j]) * float(yf[dst[i, j], c]) for j in range(k)
                     if dst[i, j] >= 0]
            exact = math.fsum(terms)
            got = float(O.bf16_to_f32(out[i:i + 1, c:c + 1])[0, 0])
            # half a bf16 ulp of the output, plus one fp32 rounding per
            # live slot of the chain
            big = max(abs(got), abs(exact), 2.0 ** -126)
            ulp = 2.0 ** (math.floor(math.log2(big)) - 7)
            assert abs(got - exact) <= (ulp / 2 + k * 2.0 ** -24 * mag[i, c]) * (1 + 1e-12)
            assert mag[i, c] == pytest.approx(math.fsum(abs(v) for v in terms))


def test_combine_single_slot_unit_weight_is_copy():
    g = np.random.Generator(np.random.PCG64(2))
    y = W.random_bf16_rows(g, 10, 64)
    dst = np.arange(10, dtype=np.int32)[::-1].reshape(10, 1).copy()
    out, _ = O.combine(y, dst, np.ones((10, 1), np.float32))
    assert np.array_equal(out, y[::-1])


def test_scaled_expert_is_exact_product():
    w = W.WORKLOADS["mixtral"]
    inp, idx, wt, L = _route_and_layout(w, 0, 64)
    out, _ = O.dispatch_bf16(inp.x, L["dst_row"], L["num_rows"])
    y = O.expert_scaled(out, L["expert_offsets"], w.experts)
    e_of_row = O.expert_of_rows(L["expert_offsets"], L["num_rows"])
    for r in range(0, L["num_rows"], 7):
        e = e_of_row[r]
        assert idx.reshape(-1)[L["src_pair"][r]] == e
        prod = O.bf16_to_f32(out[r]).astype(np.float64) * (e + 1) / w.experts
        assert np.array_equal(O.bf16_to_f32(y[r]).astype(np.float64),
                              O.bf16_to_f32(O.round_to_bf16(prod)).astype(np.float64))


def test_fp8_scale_and_multiplier_are_single_roundings():
    """scale and multiplier equal the fp64 quotients rounded once to fp32
    (exact: fp64 carries more than twice fp32's precision, so rounding the
    fp64 quotient once more gives the correctly rounded fp32 quotient)."""
    g = np.random.Generator(np.random.PCG64(4))
    x = W.random_bf16_rows(g, 64, 1024)
    x[:, ::5] = (x[:, ::5].astype(np.uint32) ^ 0x1234).astype(np.uint16)
    sc, inv = O.fp8_block_scale_inv(x)
    xf = O.bf16_to_f32(x).astype(np.float64).reshape(64, 8, 128)
    for i in range(64):
        for b in range(8):
            a = float(np.max(np.abs(xf[i, b])))
            assert sc[i, b] == np.float32(a / 448.0)
            assert inv[i, b] == np.float32(448.0 / a)


def test_fp8_codes_by_exhaustive_nearest_search():
    """Each code is the e4m3 value nearest to fp32(x * inv) (product formed
    exactly in fp64 and rounded once), found by scanning all 127 magnitudes."""
    g = np.random.Generator(np.random.PCG64(8))
    x = W.random_bf16_rows(g, 32, 512)
    codes, _ = O.quantize_fp8_blocks(x)
    _, inv = O.fp8_block_scale_inv(x)
    xf = O.bf16_to_f32(x).astype(np.float64).reshape(32, 4, 128)
    prod = (xf * inv[:, :, None].astype(np.float64)).astype(np.float32)
    table = O.e4m3_decode_table()[:0x7F]
    flat = prod.reshape(-1).astype(np.float64)
    d = np.abs(np.abs(flat)[:, None] - table[None, :])
    near = d.min(axis=1)
    mag = codes.reshape(-1) & 0x7F
    assert np.all(np.abs(table[mag] - np.abs(flat)) == near)
    assert np.all((codes.reshape(-1) >> 7) == np.signbit(flat))


def test_softmax_weights_shift_invariant_for_huge_logits():
    g = np.random.Generator(np.random.PCG64(12))
    logits = g.standard_normal((200, 16), dtype=np.float32)
    idx0, w0 = O.route_softmax_topk(logits, 4)
    idx1, w1 = O.route_softmax_topk(logits + np.float32(800.0), 4)
    assert np.all(np.isfinite(w1))
    assert np.array_equal(idx0, idx1)
    # adding 800 rounds the fp32 logits, so compare loosely
    assert np.allclose(w0, w1, rtol=0, atol=1e-3)
