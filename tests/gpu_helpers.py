"""Helpers shared by the GPU parity tests: host<->device copies and the
acceptance rules for floating-point results.

Acceptance rules (derived from the arithmetic of each step):
  * routing: expert choices equal; where they differ, the differing experts
    must be near-ties (keys within 2 fp32 ulps), which can only come from the
    fp64 sigmoid/exp of host and device rounding to different fp32 values;
    weights within 1 fp32 ulp (both sides sum in fp64 and round once).
  * combine: the oracle rounds the exact (fp64) sum S once to bf16; the GPU
    rounds an fp32 FMA chain A with |A - S| <= k * 2^-24 * sum|w y|. Two
    roundings of values that close differ by at most one bf16 ulp, plus the
    accumulation error where the terms cancel:
        |gpu - oracle| <= ulp_bf16(max(|gpu|, |oracle|)) + k * 2^-23 * sum|w y|
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


def assert_combine_close(gpu_bits, ref_bits, mag, k, what=""):
    g = O.bf16_to_f32(gpu_bits).astype(np.float64)
    r = O.bf16_to_f32(ref_bits).astype(np.float64)
    tol = ulp_bf16(np.maximum(np.abs(g), np.abs(r))) + k * 2.0 ** -23 * mag
    err = np.abs(g - r)
    bad = ~(err <= tol)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s combine mismatch at %s: gpu %r oracle %r tol %r (%d bad)"
                             % (what, tuple(i), g[tuple(i)], r[tuple(i)], tol[tuple(i)],
                                bad.sum()))
    return float((gpu_bits == ref_bits).mean()) if gpu_bits.size else 1.0


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
