"""Pins of the oracle's backward pass: weight gradients against math.fsum,
the adjoint identities of the two linear maps (<g, dispatch(x)> equals
<dispatch_backward(g), x>; <dout, combine(y)> equals <dy, y>), closed forms,
and dropped pairs."""

import math

import numpy as np

from oracle import moe_oracle as O
from synth import workloads as W


def _setup(seed, t=60, k=3, rows=200, h=48, drop=0.1):
    """Destination rows as a layout gives them: each row used by one pair."""
    g = np.random.Generator(np.random.PCG64(seed))
    dst = g.permutation(rows)[: t * k].reshape(t, k).astype(np.int32)
    dst[g.random((t, k)) < drop] = -1
    return g, dst


def test_weight_gradient_is_exact_dot_product():
    g, dst = _setup(1)
    t, k = dst.shape
    dout = W.random_bf16_rows(g, t, 48)
    y = W.random_bf16_rows(g, 200, 48)
    w = W.random_weights(g, t, k)
    dy, written, dw, dw_abs = O.combine_backward(dout, y, dst, w, 200)
    df, yf = O.bf16_to_f32(dout), O.bf16_to_f32(y)
    for i in range(t):
        for j in range(k):
            if dst[i, j] < 0:
                assert dw[i, j] == 0 and dw_abs[i, j] == 0
                continue
            terms = [float(a) * float(b) for a, b in zip(df[i], yf[dst[i, j]])]
            assert dw[i, j] == np.float32(math.fsum(terms))
            assert math.isclose(dw_abs[i, j], math.fsum(abs(v) for v in terms), rel_tol=1e-12)


def test_expert_gradient_rows_are_scaled_copies():
    g, dst = _setup(2)
    t, k = dst.shape
    dout = W.random_bf16_rows(g, t, 48)
    w = W.random_weights(g, t, k)
    dy, written, _, _ = O.combine_backward(dout, W.random_bf16_rows(g, 200, 48), dst, w, 200)
    live = dst >= 0
    assert written.sum() == live.sum()                 # one row per live pair
    df = O.bf16_to_f32(dout).astype(np.float64)
    for i, j in zip(*np.nonzero(live)):
        want = O.round_to_bf16(float(w[i, j]) * df[i])  # fp32 x bf16 is exact in fp64
        assert np.array_equal(dy[dst[i, j]], want)
    # unit weight: the gradient row is the output gradient itself
    dy1, _, _, _ = O.combine_backward(dout, W.random_bf16_rows(g, 200, 48), dst,
                                      np.ones_like(w), 200)
    for i, j in zip(*np.nonzero(live)):
        assert np.array_equal(dy1[dst[i, j]], dout[i])


def test_combine_adjoint_identity():
    """<dout, S(y)> = sum over live pairs of <w dout, y>: both sides from the
    oracle's unrounded parts (dw) and its rounded outputs within rounding."""
    g, dst = _setup(3, t=80, k=4, rows=400, h=64, drop=0.15)
    t, k = dst.shape
    dout = W.random_bf16_rows(g, t, 64)
    y = W.random_bf16_rows(g, 400, 64)
    w = W.random_weights(g, t, k)
    out, mag = O.combine(y, dst, w)
    dy, written, dw, dw_abs = O.combine_backward(dout, y, dst, w, 400)
    lhs = (O.bf16_to_f32(dout).astype(np.float64) * O.bf16_to_f32(out)).sum()
    # sum_t sum_j w dw equals <dout, exact combine>
    rhs = float((w.astype(np.float64) * dw.astype(np.float64)).sum())
    mid = (O.bf16_to_f32(dy[written]).astype(np.float64) *
           O.bf16_to_f32(y[written]).astype(np.float64)).sum()
    bound = 2.0 ** -8 * (np.abs(O.bf16_to_f32(dout)).astype(np.float64) * mag).sum()
    assert abs(lhs - rhs) <= bound + 1e-3
    assert abs(mid - rhs) <= 2.0 ** -8 * (w[dst >= 0].astype(np.float64) * dw_abs[dst >= 0]).sum() + 1e-3


def test_dispatch_adjoint_and_closed_form():
    g = np.random.Generator(np.random.PCG64(4))
    t, k, h = 50, 4, 32
    idx = W.random_topk_idx(g, t, 16, k, mask_frac=0.1)
    L = O.layout(idx, 16, 4, 0)
    x = W.random_bf16_rows(g, t, h)
    rows_x, written = O.dispatch_bf16(x, L["dst_row"], L["num_rows"])
    grows = W.random_bf16_rows(g, L["num_rows"], h)
    dx, mag = O.dispatch_backward(grows, L["dst_row"])
    xf = O.bf16_to_f32(x).astype(np.float64)
    lhs = (O.bf16_to_f32(grows[written]).astype(np.float64) * O.bf16_to_f32(rows_x[written])).sum()
    rhs = (O.bf16_to_f32(dx).astype(np.float64) * xf).sum()
    assert abs(lhs - rhs) <= 2.0 ** -8 * (mag * np.abs(xf)).sum() + 1e-6
    # gradients equal to the dispatched rows themselves: dx = bf16(live_k * x)
    dx2, _ = O.dispatch_backward(rows_x, L["dst_row"])
    nlive = (L["dst_row"] >= 0).sum(axis=1).astype(np.float64)
    assert np.array_equal(dx2, O.round_to_bf16(xf * nlive[:, None]))
