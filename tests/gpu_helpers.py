"""Helpers shared by the GPU parity tests: host<->device copies and the
acceptance rules for floating-point results.

Acceptance rules (derived from the arithmetic of each step):
  * routing: expert choices equal; where they differ, the differing experts
    must be near-ties (keys within 2 fp32 ulps), which can only come from the
    fp64 sigmoid/exp of host and device rounding to different fp32 values;
    weights within 1 fp32 ulp (both sides sum in fp64 and round once).
  * combine (and the gradient of dispatch, and both levels of the
    hierarchical combine): the oracle runs the combine's own arithmetic, an
    fp32 chain of fused multiply-adds in slot order from +0 rounded once to
    bf16, so the GPU's bits must equal the oracle's. (The contract's bound is
    one bf16 ulp; the failure message reports the largest distance in ulps.)
    Every checked case is recorded with its element count, and the session
    writes the list to combine_exactness.txt in the folder MOE_TEST_LOG_DIR
    names (when set).
"""

from __future__ import annotations

import numpy as np
import torch

from oracle import moe_oracle as O


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def poison_like(shape, dtype) -> torch.Tensor:
    """Device tensor filled with 0xFF bytes (detects rows that should stay
    untouched and rows that were never written)."""
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)
    return t


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(v.astype(np.float64))
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -126)
    return np.ldexp(1.0, e - 7)


EXACT_LOG: list = []


def bf16_ulp_distance(a_bits, b_bits) -> np.ndarray:
    """Number of bf16 values between two bf16 patterns (0 when equal; +0 and
    -0 count as equal): distance of their positions on the ordered line."""
    def order(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(order(a_bits) - order(b_bits))


def assert_combine_exact(gpu_bits, ref_bits, what=""):
    """GPU combine output equal to the oracle's bit for bit."""
    gpu_bits = np.asarray(gpu_bits).view(np.uint16)
    ref_bits = np.asarray(ref_bits).view(np.uint16)
    assert gpu_bits.shape == ref_bits.shape, (what, gpu_bits.shape, ref_bits.shape)
    bad = gpu_bits != ref_bits
    if bad.any():
        dist = bf16_ulp_distance(gpu_bits, ref_bits)
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(
            "%s combine differs from the oracle at %d of %d outputs (largest distance %d "
            "bf16 ulps); first at %s: gpu 0x%04x oracle 0x%04x"
            % (what, int(bad.sum()), bad.size, int(dist.max()), i, gpu_bits[i], ref_bits[i]))
    EXACT_LOG.append((what, int(gpu_bits.size)))
    return 1.0


def assert_route_close(idx_g, w_g, idx_o, w_o, key, what=""):
    """key: the oracle's fp32 selection keys (masked experts included)."""
    diff_rows = np.nonzero((idx_g != idx_o).any(axis=1))[0]
    for t in diff_rows:
        a, b = set(idx_g[t].tolist()), set(idx_o[t].tolist())
        if a == b:
            # same set, different slot order: the swapped keys must tie
            pairs = zip(idx_g[t], idx_o[t])
        else:
            pairs = zip(sorted(a - b), sorted(b - a))
        for eg, eo in pairs:
            kg, ko = np.float32(key[t, eg]), np.float32(key[t, eo])
            gap = abs(float(kg) - float(ko))
            assert gap <= 2 * float(np.spacing(max(abs(kg), abs(ko)))), (
                "%s token %d: experts %s vs %s are not a near-tie" % (what, t, idx_g[t], idx_o[t]))
    same = np.setdiff1d(np.arange(len(idx_g)), diff_rows)
    wg, wo = w_g[same], w_o[same]
    assert np.all(np.abs(wg - wo) <= np.spacing(np.maximum(np.abs(wg), np.abs(wo)))), what
    return len(diff_rows)


def assert_bf16_within_ulp(gpu_bits, ref_bits, what=""):
    """One bf16 ulp: the GPU rounds an fp32 product to bf16, the oracle rounds
    the exact product once (the two roundings can differ by one step)."""
    g = O.bf16_to_f32(gpu_bits).astype(np.float64)
    r = O.bf16_to_f32(ref_bits).astype(np.float64)
    bad = ~(np.abs(g - r) <= ulp_bf16(np.maximum(np.abs(g), np.abs(r))))
    assert not bad.any(), "%s: %d values differ by more than one bf16 ulp" % (what, bad.sum())
    return float((gpu_bits == ref_bits).mean()) if gpu_bits.size else 1.0


def dot_tolerance(hidden, ref, dw_abs):
    """Bound for an fp32 dot product of `hidden` terms summed as the kernel
    does (per-lane FMA chains of at most 32 terms per group, a 6-level wave
    tree, one add per group and a 4-wave sum): n * 2^-24 * sum|terms| with
    n = 48 + groups, plus the final fp32 rounding of the reference."""
    groups = -(-(hidden // 8) // 1024)
    return (48 + groups) * 2.0 ** -24 * dw_abs + 2.0 ** -24 * np.abs(ref)
