"""GPU parity: the HIP path through the C ABI against the CPU oracle, element
by element, on the same seeded inputs.

Bars: bit-exact for expert choices (up to logged near-ties of the fp64
transcendentals), layout outputs, bf16 rows and FP8 codes/scales; routing
weights within 1 fp32 ulp; combine outputs equal to the oracle's bits (the
oracle runs the combine's fp32 slot-order chain; the contract's bound is one
bf16 ulp). Full-size layers take the FP8 codes and the combine from the
oracle's C twin, pinned bit for bit to the numpy oracle. Output buffers are pre-filled with 0xFF and
followed by guard rows, so unwritten rows and stray writes are caught.
"""

import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import combine_moe_layout_06_amd as M  # noqa: E402
from combine_moe_layout_06_amd import LayerBuffers  # noqa: E402
from gpu_helpers import (assert_bf16_within_ulp, assert_combine_exact,  # noqa: E402
                         assert_route_close, dev, dot_tolerance, host, poison_like)
from oracle import c_twin as C  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from synth import workloads as W  # noqa: E402

GUARD = 8  # guard rows after every row buffer
LAYOUT_POISON = 0x7B7B7B7B   # no row, pair index or count takes this value


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("the GPU tests need a visible MI355X")
    M.lib()   # raises loudly if the HIP library is missing
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ route

def oracle_keys(logits, bias, score_fn):
    s = O._sigmoid_f32(logits) if score_fn == 1 else logits.astype(np.float32)
    return O._selection_key(s, bias)


def gpu_route(logits, bias, k, score_fn, G, kg):
    t, e = logits.shape
    idx = poison_like((max(t, 1), k), torch.int32)
    w = poison_like((max(t, 1), k), torch.float32)
    M.moe_route(t, e, k, dev(logits) if t else None, dev(bias) if bias is not None else None,
                score_fn, G, kg, idx, w)
    return host(idx)[:t], host(w)[:t]


def _logits(g, t, e, kind):
    if kind == "int":      # small integers: many exact ties
        return g.integers(-3, 4, size=(t, e)).astype(np.float32)
    if kind == "const":    # every key equal: the tie order alone decides
        return np.full((t, e), 0.25, dtype=np.float32)
    return g.standard_normal((t, e), dtype=np.float32)


ROUTE_CASES = [
    # T, E, k, score, G, kg, bias, logits
    (128, 8, 2, 0, 1, 1, None, "normal"),
    (16384, 8, 2, 0, 1, 1, None, "normal"),
    (4096, 256, 8, 1, 8, 4, "normal", "normal"),
    (8192, 128, 8, 0, 1, 1, "zipf", "normal"),
    (1001, 12, 3, 0, 1, 1, None, "int"),
    (515, 64, 6, 1, 8, 3, "int", "int"),
    (333, 512, 32, 1, 16, 8, "normal", "normal"),
    (77, 6, 1, 0, 1, 1, "normal", "normal"),
    (300, 96, 4, 1, 1, 1, "normal", "normal"),
    (200, 16, 3, 1, 16, 4, None, "normal"),
    (130, 200, 7, 1, 5, 2, "normal", "normal"),
    (3, 256, 8, 1, 8, 4, "normal", "normal"),
    (0, 256, 8, 1, 8, 4, None, "normal"),
    # 16-lane teams: 1, 2 and 4 slots per group, k = team size
    (999, 128, 16, 1, 2, 1, "normal", "normal"),
    (517, 128, 8, 1, 4, 2, "normal", "normal"),
    (700, 128, 6, 1, 8, 5, "normal", "normal"),
    (333, 64, 8, 1, 2, 1, "int", "int"),
    (600, 128, 16, 0, 1, 1, None, "normal"),
    (450, 192, 8, 1, 6, 3, "int", "int"),
    # k above the team size falls back to one wave per token
    (300, 64, 10, 0, 1, 1, None, "normal"),
    (301, 40, 9, 1, 1, 1, "normal", "normal"),
    # one wave per token, consecutive slots per lane: groups of 1, 8, 16 and
    # 32 lanes, the LDS path, softmax with exact ties across and within
    # lanes, rows that do not fill the last lane (scalar loads), G = 64
    (257, 512, 32, 1, 64, 8, "normal", "normal"),
    (150, 256, 8, 1, 64, 16, "normal", "normal"),
    (210, 512, 16, 1, 8, 3, "normal", "normal"),
    (200, 256, 6, 1, 4, 2, "int", "int"),
    (180, 256, 4, 1, 2, 1, "normal", "normal"),
    (190, 130, 5, 1, 13, 3, "normal", "normal"),
    (300, 256, 8, 0, 1, 1, None, "normal"),
    (250, 256, 8, 0, 1, 1, None, "int"),
    (220, 512, 32, 0, 1, 1, "int", "int"),
    (129, 131, 7, 1, 1, 1, "normal", "normal"),
    # all logits equal, no bias: the lowest groups, then the lowest experts
    (64, 256, 8, 1, 8, 4, None, "const"),
    (33, 512, 32, 1, 16, 8, None, "const"),
    (40, 256, 8, 0, 1, 1, None, "const"),
    (70, 128, 8, 1, 4, 2, None, "const"),
]


@pytest.mark.parametrize("case", ROUTE_CASES, ids=lambda c: "T%d_E%d_k%d_f%d_G%d" % c[:5])
def test_route_parity(case):
    t, e, k, fn, G, kg, bias_kind, lk = case
    say("route case", case)
    g = np.random.Generator(np.random.PCG64(t * 7 + e))
    logits = _logits(g, t, e, lk)
    bias = None
    if bias_kind == "normal":
        bias = (g.standard_normal(e, dtype=np.float32) * np.float32(0.1)).astype(np.float32)
    elif bias_kind == "zipf":
        bias = W.zipf_bias(g, e)
    elif bias_kind == "int":
        bias = (g.integers(-1, 2, size=e) * 0.125).astype(np.float32)
    idx_g, w_g = gpu_route(logits, bias, k, fn, G, kg)
    idx_o, w_o = O.route(logits, k, fn, G, kg, bias)
    nd = assert_route_close(idx_g, w_g, idx_o, w_o, oracle_keys(logits, bias, fn), str(case))
    say("  tokens with a near-tie difference:", nd)
    if fn == 0 or lk in ("int", "const"):
        assert nd == 0   # no transcendental decides these choices
    if lk == "const" and bias_kind is None:
        # keys all equal: groups 0..kg-1 are kept and the experts come in index order
        assert (idx_g == np.arange(k, dtype=np.int32)[None, :]).all()
    assert idx_g.dtype == np.int32 and ((idx_g >= 0) & (idx_g < e)).all()


# ----------------------------------------------------------------- layout

def gpu_layout(idx, E, R, cap, with_rtc=True):
    t, k = idx.shape
    rows = E * cap if cap else t * k
    b = LayerBuffers(t, 8, E, k, R, cap, M.MOE_DTYPE_BF16)
    b.expert_counts = poison_like(E, torch.int32)
    b.expert_offsets = poison_like(E + 1, torch.int32)
    b.rank_counts = poison_like(R, torch.int32)
    b.rank_offsets = poison_like(R + 1, torch.int32)
    b.rank_token_counts = poison_like(R, torch.int32) if with_rtc else None
    # dst_row and src_pair hold -1 for masked pairs and empty rows: poisoned
    # with another value, so that an entry the layout fails to write shows
    b.dst_row = torch.full((max(t, 1), k), LAYOUT_POISON, dtype=torch.int32, device="cuda")
    src_full = torch.full((rows + GUARD,), LAYOUT_POISON, dtype=torch.int32, device="cuda")
    b.src_pair = src_full
    b.overflow = poison_like(1, torch.int32)
    b.workspace_bytes = M.moe_layout_workspace_bytes(t, E, k)
    b.workspace = torch.empty(max(b.workspace_bytes, 4), dtype=torch.uint8, device="cuda")
    b.topk_idx = dev(idx) if t else None
    b.layout()
    src = host(src_full)
    assert np.all(src[rows:] == LAYOUT_POISON), "stray write after src_pair"
    out = dict(expert_counts=host(b.expert_counts), expert_offsets=host(b.expert_offsets),
               rank_counts=host(b.rank_counts), rank_offsets=host(b.rank_offsets),
               dst_row=host(b.dst_row)[:t], src_pair=src[:rows], overflow=host(b.overflow))
    if with_rtc:
        out["rank_token_counts"] = host(b.rank_token_counts)
    return out


LAYOUT_CASES = [
    # T, E, k, R, cap, distinct, mask_frac
    (128, 8, 2, 4, 0, True, 0.0),
    (16384, 8, 2, 8, 0, True, 0.0),
    (4096, 256, 8, 32, 0, True, 0.0),
    (8192, 128, 8, 16, 0, True, 0.0),
    (128, 256, 8, 32, 128, True, 0.0),
    (129, 8, 8, 2, 0, True, 0.0),           # ragged last tile
    (1000, 6, 4, 3, 0, False, 0.1),         # duplicates inside a token, masked slots
    (513, 64, 2, 64, 7, False, 0.3),        # capacity with drops
    (1, 512, 32, 16, 0, True, 0.0),
    (2000, 512, 32, 512, 1, True, 0.05),    # max experts and top-k
    (300, 1, 1, 1, 0, True, 0.0),           # a single expert
    (0, 8, 2, 4, 0, True, 0.0),             # empty, packed
    (0, 8, 2, 4, 3, True, 0.0),             # empty, capacity
    (777, 20, 6, 5, 50, True, 1.0),         # every slot masked
    (4097, 256, 8, 32, 0, True, 0.0),       # one token past 32 tiles
    (4000, 96, 8, 48, 0, True, 0.0),        # R not a power of two, E/R = 2
    (32768, 512, 1, 512, 0, True, 0.0),     # k = 1, 512 ranks
    # many tiles: up to 64 tiles of E = 256 the place blocks stage the whole
    # histogram, beyond that (or from 256 tiles) a scan pass feeds them
    (8191, 256, 8, 32, 0, True, 0.0),       # 64 tiles, ragged: staged
    (8300, 256, 8, 32, 0, True, 0.0),       # 65 tiles, ragged: scanned
    (65613, 256, 8, 32, 0, True, 0.02),     # 513 tiles, masked slots
    (131073, 8, 2, 4, 0, True, 0.0),        # 257 tiles of 512 tokens
    (70000, 64, 4, 8, 4300, False, 0.1),    # 274 tiles, capacity with drops
    (2100, 512, 32, 512, 0, True, 0.05),    # 66 tiles, 512 ranks
    (2100, 512, 32, 16, 5, True, 0.0),      # more fill blocks than tiles
    # one tile, 1024-thread blocks: every wave holds one 64-pair chunk
    (1024, 16, 1, 4, 0, True, 0.0),         # a full tile, k = 1
    (512, 128, 2, 64, 0, True, 0.0),        # rank token counts per token (no bitmasks)
    (100, 6, 4, 3, 0, False, 0.1),          # duplicates, masked slots
    (200, 64, 5, 8, 3, False, 0.2),         # 1000 pairs, drops
    (8, 512, 8, 64, 64, True, 0.0),         # 32 blocks mark unused rows
    (7, 8, 3, 2, 0, True, 0.0),             # 21 pairs
    (64, 512, 16, 1, 0, True, 0.0),         # one rank owns all 512 experts
]


@pytest.mark.parametrize("case", LAYOUT_CASES, ids=lambda c: "T%d_E%d_k%d_R%d_cap%d" % c[:5])
def test_layout_parity(case):
    t, e, k, r, cap, distinct, mf = case
    say("layout case", case)
    g = np.random.Generator(np.random.PCG64(sum(case[:5]) + 17))
    idx = W.random_topk_idx(g, t, e, k, distinct=distinct, mask_frac=mf)
    got = gpu_layout(idx, e, r, cap)
    want = O.layout(idx, e, r, cap)
    for name, val in got.items():
        assert np.array_equal(val, want[name].reshape(val.shape)), (case, name)


def test_layout_skewed_and_single_expert():
    t, e, k = 5000, 128, 8
    g = np.random.Generator(np.random.PCG64(3))
    idx = W.random_topk_idx(g, t, e, k)
    idx[: t // 2, 0] = 5                       # half the tokens pick expert 5 first
    idx[: t // 2, 1:] = np.where(idx[: t // 2, 1:] == 5, 6, idx[: t // 2, 1:])
    for cap in (0, 100):
        got = gpu_layout(idx, e, 16, cap)
        want = O.layout(idx, e, 16, cap)
        for name, val in got.items():
            assert np.array_equal(val, want[name].reshape(val.shape)), (cap, name)


def test_layout_ignores_out_of_range_ids():
    g = np.random.Generator(np.random.PCG64(4))
    idx = W.random_topk_idx(g, 400, 16, 4)
    junk = idx.copy()
    junk[::7, 1] = 16
    junk[::11, 2] = -5
    junk[::13, 0] = 1 << 30
    got = gpu_layout(junk, 16, 4, 0)
    clean = np.where((junk >= 0) & (junk < 16), junk, -1).astype(np.int32)
    want = O.layout(clean, 16, 4, 0)
    for name, val in got.items():
        assert np.array_equal(val, want[name].reshape(val.shape)), name


@pytest.mark.parametrize("t,k", [(200, 4), (900, 4), (33000, 8)], ids=["one_tile", "staged", "scanned"])
def test_layout_without_rank_token_counts(t, k):
    g = np.random.Generator(np.random.PCG64(5))
    idx = W.random_topk_idx(g, t, 32, k)
    got = gpu_layout(idx, 32, 8, 0, with_rtc=False)
    want = O.layout(idx, 32, 8, 0)
    for name, val in got.items():
        assert np.array_equal(val, want[name].reshape(val.shape)), name


# --------------------------------------------------------------- dispatch

def gpu_dispatch(x, dst, num_rows, fp8):
    assert x.dtype == np.uint16 and dst.dtype == np.int32
    t, h = x.shape
    k = dst.shape[1]
    if fp8:
        out_full = poison_like((num_rows + GUARD, h), torch.uint8)
        sc_full = poison_like((num_rows + GUARD, h // 128), torch.float32)
    else:
        out_full = poison_like((num_rows + GUARD, h), torch.int16)
        sc_full = None
    M.moe_dispatch(t, h, k, num_rows, dev(x) if t else None, dev(dst) if t else None,
                   M.MOE_DTYPE_FP8_E4M3 if fp8 else M.MOE_DTYPE_BF16, out_full,
                   sc_full, None)
    out = host(out_full, np.uint8 if fp8 else np.uint16)
    poison = 0xFF if fp8 else 0xFFFF
    assert np.all(out[num_rows:] == poison), "stray write after the dispatch buffer"
    if fp8:
        sc = host(sc_full).view(np.uint32)
        assert np.all(sc[num_rows:] == 0xFFFFFFFF), "stray write after the scales"
        return out[:num_rows], sc[:num_rows].view(np.float32)
    return out[:num_rows], None


DISPATCH_CASES = [
    # T, H, k, E, cap, fp8
    (128, 256, 2, 8, 0, False),
    (300, 520, 3, 10, 0, False),       # 65 chunks: ragged wave tail
    (1500, 4096, 2, 8, 0, False),
    (257, 7168, 8, 256, 0, True),
    (64, 128, 4, 16, 0, True),
    (100, 384, 2, 8, 0, True),          # 3 blocks: partial 512-column step
    (33, 896, 5, 12, 3, True),          # capacity with drops, FP8
    (40, 33280, 2, 4, 0, True),         # 260 blocks: more than one part per row
    (500, 1152, 4, 16, 0, True),        # 9 blocks: two steps, the second of one block
    (77, 8320, 3, 8, 0, True),          # 65 blocks, 9 steps: two parts of 5 steps
    (200, 16384, 8, 64, 0, True),       # 16 steps: two parts of 8
    (9000, 1024, 1, 4, 0, False),
    (0, 256, 2, 8, 0, False),
    (0, 256, 2, 8, 0, True),
]


@pytest.mark.parametrize("case", DISPATCH_CASES, ids=lambda c: "T%d_H%d_k%d_E%d_cap%d_fp8%d" % c)
def test_dispatch_parity(case):
    t, h, k, e, cap, fp8 = case
    say("dispatch case", case)
    g = np.random.Generator(np.random.PCG64(t + h + k))
    x = W.random_bf16_rows(g, t, h)
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.05)
    L = O.layout(idx, e, max(1, e // 2) if e % 2 == 0 else 1, cap)
    rows = L["num_rows"]
    out, sc = gpu_dispatch(x, L["dst_row"], rows, fp8)
    if fp8:
        q, s, written = O.dispatch_fp8(x, L["dst_row"], rows)
        assert np.array_equal(out[written], q[written])
        assert np.array_equal(sc[written].view(np.uint32), s[written].view(np.uint32))
        assert np.all(out[~written] == 0xFF)
        assert np.all(sc[~written].view(np.uint32) == 0xFFFFFFFF)
    else:
        o, written = O.dispatch_bf16(x, L["dst_row"], rows)
        assert np.array_equal(out[written], o[written])
        assert np.all(out[~written] == 0xFFFF)


def test_fp8_every_bf16_pattern_at_several_scales():
    """All finite bf16 patterns, in blocks whose amax is set by a chosen
    extreme element, so every pattern is quantised at several multipliers."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = O.bf16_to_f32(bits)
    bits = bits[np.isfinite(f)]
    rows = []
    for big in (0x43E0, 0x4000, 0x3F80, 0x7F7F, 0x0080, 0x0001, 0x5A5A):   # 448, 2, 1, max, min normal, min subnormal, misc
        v = bits.copy()
        v = np.concatenate([v, np.zeros((-len(v)) % 127, np.uint16)]).reshape(-1, 127)
        blocks = np.concatenate([np.full((len(v), 1), big, np.uint16), v], axis=1)
        rows.append(blocks.reshape(-1))
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros((-len(x)) % 1024, np.uint16)]).reshape(-1, 1024)
    t = x.shape[0]
    dst = np.arange(t, dtype=np.int32).reshape(t, 1)
    out, sc = gpu_dispatch(x, dst, t, True)
    q, s = O.quantize_fp8_blocks(x)
    assert np.array_equal(out, q)
    assert np.array_equal(sc.view(np.uint32), s.view(np.uint32))


def test_fp8_exact_ties_round_to_even():
    """Blocks whose amax is 448 quantise with multiplier 1, so bf16 inputs
    that are e4m3 midpoints are exact ties."""
    table = O.e4m3_decode_table()[:0x7F]
    mids = ((table[:-1] + table[1:]) / 2).astype(np.float32)
    mb = (mids.view(np.uint32) >> 16).astype(np.uint16)
    exact = O.bf16_to_f32(mb).astype(np.float64) == (table[:-1] + table[1:]) / 2
    mb = mb[exact]
    blk = np.concatenate([np.array([0x43E0], np.uint16), mb, (mb | 0x8000)])
    blk = np.concatenate([blk, np.zeros((-len(blk)) % 128, np.uint16)])
    x = blk.reshape(1, -1)
    x = np.concatenate([x, np.zeros((1, (-x.shape[1]) % 128), np.uint16)], axis=1)
    out, sc = gpu_dispatch(x, np.zeros((1, 1), np.int32), 1, True)
    q, s = O.quantize_fp8_blocks(x)
    assert np.array_equal(out, q) and np.array_equal(sc, s)


# ---------------------------------------------------------------- combine

def gpu_combine(y, dst, w, t, h):
    assert y.dtype == np.uint16 and dst.dtype == np.int32 and w.dtype == np.float32
    k = dst.shape[1]
    out_full = poison_like((max(t, 1) + GUARD, h), torch.int16)
    M.moe_combine(t, h, k, y.shape[0], dev(y) if y.shape[0] else None,
                  dev(dst) if t else None, dev(w) if t else None, out_full)
    out = host(out_full, np.uint16)
    assert np.all(out[max(t, 1):] == 0xFFFF), "stray write after the combine output"
    return out[:t]


COMBINE_CASES = [
    # T, H, k, rows, drop_frac
    (128, 256, 2, 256, 0.0),
    (1000, 520, 3, 3000, 0.1),
    (4096, 7168, 8, 32768, 0.0),
    # k = 8, rows of 7 parts of 2 KiB, 8..16 items per wave: outputs held in registers
    (2100, 7168, 8, 16800, 0.05),        # 8 items per wave, the last wave short
    (3000, 7040, 8, 24000, 0.1),         # 11 items; each row's last part is 112 chunks
    (4097, 7168, 8, 32776, 0.0),         # 15 items
    (4600, 7168, 8, 36800, 0.02),        # 16 items
    (8192, 4096, 8, 65536, 0.02),        # rows of 4 parts: the per-item kernel
    (777, 4096, 6, 5000, 0.2),
    (500, 1024, 4, 2000, 0.0),
    (300, 2048, 1, 300, 0.0),
    (200, 512, 11, 3000, 0.1),           # k without a specialised kernel
    (64, 1024, 32, 2048, 0.5),
    (0, 256, 2, 0, 0.0),
]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=lambda c: "T%d_H%d_k%d_rows%d" % c[:4])
def test_combine_parity(case):
    t, h, k, rows, drop = case
    say("combine case", case)
    g = np.random.Generator(np.random.PCG64(t * 3 + h + k))
    y = W.random_bf16_rows(g, rows, h)
    if t:
        dst = np.stack([g.choice(rows, size=k, replace=False) for _ in range(t)]).astype(np.int32)
        dst[g.random((t, k)) < drop] = -1
    else:
        dst = np.zeros((0, k), np.int32)
    w = W.random_weights(g, t, k)
    got = gpu_combine(y, dst, w, t, h)
    want, _ = O.combine(y, dst, w)
    assert_combine_exact(got, want, "combine %s" % (case,))


def _rounding_weights():
    """fp32 values whose bf16 rounding covers every exponent (subnormals and the largest
    binade included), both signs, the low 16 bits below, at and above the halfway point, kept
    bits even and odd and all ones (a carry into the exponent, up to infinity), and the two
    infinities. NaN is left out: its bits are not part of the contract."""
    lows = (0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF)
    kept = (0x00, 0x01, 0x7E, 0x7F)
    pats = [(sign << 31) | (e << 23) | (m << 16) | lo
            for sign in (0, 1) for e in range(255) for m in kept for lo in lows]
    pats += [0x7F800000, 0xFF800000]
    return np.array(pats, dtype=np.uint32).view(np.float32)


def test_combine_rounds_every_binade_like_the_oracle():
    """With k = 1 and expert rows of 1.0 the fp32 accumulator is the weight itself, so the
    output is the weight's bf16 rounding: compared with the oracle on every binade and
    rounding boundary (the per-item kernel)."""
    w = _rounding_weights()
    t, h = len(w), 8
    y = np.full((t, h), 0x3F80, np.uint16)                   # bf16 1.0
    dst = np.arange(t, dtype=np.int32).reshape(t, 1)
    got = gpu_combine(y, dst, w.reshape(t, 1), t, h)
    want, _ = O.combine(y, dst, w.reshape(t, 1))
    assert np.array_equal(got, want)
    # the sum starts from +0.0, so -0.0 comes out as +0.0
    assert np.array_equal(want[:, 0], O.round_to_bf16(w.astype(np.float64) + 0.0))


def test_held_combine_rounds_every_binade_like_the_oracle():
    """The same rounding cases through the held-output kernel (k = 8, rows of 7 parts,
    3000 tokens: 11 items per wave): slot 0 carries the weight, the other seven weigh 0."""
    w = _rounding_weights()
    t, h, k = 3000, 7168, 8
    y = np.full((k, h), 0x3F80, np.uint16)
    dst = np.tile(np.arange(k, dtype=np.int32), (t, 1))
    for start in range(0, len(w), t):
        part = np.resize(w[start:start + t], t)               # the last call repeats values
        wt = np.zeros((t, k), np.float32)
        wt[:, 0] = part
        got = gpu_combine(y, dst, wt, t, h)
        want, _ = O.combine(y, dst, wt)
        assert np.array_equal(got, want), "calls from weight %d" % start


def test_combine_ignores_rows_past_num_rows():
    g = np.random.Generator(np.random.PCG64(6))
    y = W.random_bf16_rows(g, 50, 256)
    dst = g.integers(0, 50, size=(40, 2)).astype(np.int32)
    dst[::3, 1] = 50 + 1000                     # out of range: skipped like a drop
    w = W.random_weights(g, 40, 2)
    got = gpu_combine(y, dst, w, 40, 256)
    want, _ = O.combine(y, np.where(dst < 50, dst, -1).astype(np.int32), w)
    assert_combine_exact(got, want)


# ------------------------------------------------------------ whole layer

def run_layer_gpu(w, inp):
    t = inp.x.shape[0]
    b = LayerBuffers.allocate(t, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                              w.dispatch_dtype == W.DTYPE_FP8_E4M3)
    logits = dev(inp.logits)
    bias = dev(inp.bias) if inp.bias is not None else None
    x = dev(inp.x)
    M.run_layer(b, logits, bias, x, w.score_fn, w.groups, w.topk_groups)
    torch.cuda.synchronize()
    return b


def fake_expert(w, L, x, dispatched, twin=False):
    """Stand-in expert on the oracle side (harness, not the method)."""
    if w.expert_kind == "identity":
        return dispatched
    if w.expert_kind == "scaled":
        return O.expert_scaled(dispatched, L["expert_offsets"], w.experts)
    codes, sc = (C if twin else O).quantize_fp8_blocks(x)   # one row per token
    y_tok = O.expert_dequant(codes, sc)
    y, _ = O.dispatch_bf16(y_tok, L["dst_row"], L["num_rows"])
    return y


# Full-size layers of every headline shape over seeds 0..4, the reduced
# dsv3 layer and the tiny and decode layers. Layers of at least 2^22 input
# elements take the FP8 codes and the combine from the oracle's C twin.
LAYER_CASES = ([("tiny", 0, None), ("tiny", 1, None)]
               + [(n, s, None) for n in ("mixtral", "dsv3", "qwen3_skew") for s in range(5)]
               + [("dsv3", 3, 1000), ("decode", 1000, None), ("decode", 1001, None),
                  ("decode", 1002, None)])


@pytest.mark.parametrize("name,seed,tokens", LAYER_CASES)
def test_layer_end_to_end(name, seed, tokens):
    w = W.WORKLOADS[name]
    say("layer", name, "seed", seed)
    inp = W.make_inputs(w, seed, tokens=tokens)
    t = inp.x.shape[0]
    twin = inp.x.size >= 1 << 22
    b = run_layer_gpu(w, inp)
    idx_g, w_g = host(b.topk_idx), host(b.topk_weights)
    idx_o, w_o = O.route(inp.logits, w.top_k, w.score_fn, w.groups, w.topk_groups, inp.bias)
    nd = assert_route_close(idx_g, w_g, idx_o, w_o, oracle_keys(inp.logits, inp.bias, w.score_fn))
    say("  route ok; near-tie tokens:", nd)
    # downstream steps are checked on the GPU's own routing
    L = O.layout(idx_g, w.experts, w.ranks, w.capacity)
    for name_ in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets",
                  "rank_token_counts", "src_pair", "overflow"):
        got = host(getattr(b, name_))
        want = L[name_]
        assert np.array_equal(got[:want.size].reshape(want.shape), want), name_
    assert np.array_equal(host(b.dst_row), L["dst_row"])
    assert int(host(b.expert_counts).sum()) == t * w.top_k
    say("  layout ok; overflow", int(L["overflow"][0]))
    rows = L["num_rows"]
    if b.fp8:
        got_q = host(b.dispatched)[:rows]
        got_s = host(b.scales)[:rows]
        if twin:
            q_tok, s_tok = C.quantize_fp8_blocks(inp.x)
            d = L["dst_row"].reshape(-1)
            live = d >= 0
            tok = np.repeat(np.arange(t), w.top_k)[live]
            assert np.array_equal(got_q[d[live]], q_tok[tok])
            assert np.array_equal(got_s[d[live]].view(np.uint32), s_tok[tok].view(np.uint32))
            oracle_out = None
        else:
            q, s, written = O.dispatch_fp8(inp.x, L["dst_row"], rows)
            assert np.array_equal(got_q[written], q[written])
            assert np.array_equal(got_s[written].view(np.uint32), s[written].view(np.uint32))
            oracle_out = q
    else:
        o, written = O.dispatch_bf16(inp.x, L["dst_row"], rows)
        got_o = host(b.dispatched, np.uint16)[:rows]
        assert np.array_equal(got_o[written], o[written])
        oracle_out = o
    say("  dispatch ok")
    y = fake_expert(w, L, inp.x, oracle_out, twin)
    y_dev = dev(np.ascontiguousarray(y))
    b.combine(y_dev)
    got_c = host(b.combined, np.uint16)[:t]
    want_c = C.combine(y, L["dst_row"], w_g) if twin else O.combine(y, L["dst_row"], w_g)[0]
    assert_combine_exact(got_c, want_c, "layer %s seed %d T=%d" % (name, seed, t))
    say("  combine ok: equal to the oracle's bits")
    if w.expert_kind == "identity" and w.capacity == 0:
        # the round trip returns x (as values: a sum that starts at +0 turns
        # an input of -0 into +0)
        assert np.array_equal(O.bf16_to_f32(got_c), O.bf16_to_f32(inp.x))


def test_layer_is_deterministic():
    w = W.WORKLOADS["dsv3"]
    inp = W.make_inputs(w, 2, tokens=2048)
    a = run_layer_gpu(w, inp)
    b = run_layer_gpu(w, inp)
    for name in ("topk_idx", "topk_weights", "dst_row", "src_pair", "expert_counts",
                 "rank_token_counts", "dispatched", "scales"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


# ------------------------------------------------------------------ MXFP8

def gpu_dispatch_mx(x, dst, num_rows):
    assert x.dtype == np.uint16 and dst.dtype == np.int32
    t, h = x.shape
    k = dst.shape[1]
    out_full = poison_like((num_rows + GUARD, h), torch.uint8)
    sc_full = poison_like((num_rows + GUARD, h // 32), torch.uint8)
    M.moe_dispatch(t, h, k, num_rows, dev(x) if t else None, dev(dst) if t else None,
                   M.MOE_DTYPE_MXFP8_E4M3, out_full, sc_full, None)
    out, sc = host(out_full), host(sc_full)
    assert np.all(out[num_rows:] == 0xFF) and np.all(sc[num_rows:] == 0xFF), "stray write"
    return out[:num_rows], sc[:num_rows]


MX_CASES = [
    # T, H, k, E, cap
    (257, 7168, 8, 256, 0),
    (100, 96, 2, 8, 0),              # 3 blocks: partial 16-block step
    (33, 1056, 5, 12, 3),            # capacity with drops; 33 blocks
    (40, 33280, 2, 4, 0),            # 1040 blocks: several parts per row
    (1500, 4096, 2, 8, 0),
    (64, 8704, 3, 8, 0),             # 17 steps: two parts of 9 (the 14-step instance)
    (90, 16384, 4, 16, 0),           # 32 steps: two parts of 16
    (200, 1536, 8, 32, 0),           # 3 steps (the 4-step instance)
    (10, 32, 1, 2, 0),               # one block
    (0, 256, 2, 8, 0),
]


@pytest.mark.parametrize("case", MX_CASES, ids=lambda c: "T%d_H%d_k%d_E%d_cap%d" % c)
def test_dispatch_mxfp8_parity(case):
    t, h, k, e, cap = case
    say("mxfp8 dispatch case", case)
    g = np.random.Generator(np.random.PCG64(t + 3 * h + k))
    x = W.random_bf16_rows(g, t, h)
    idx = W.random_topk_idx(g, t, e, k, mask_frac=0.05)
    L = O.layout(idx, e, 1, cap)
    rows = L["num_rows"]
    out, sc = gpu_dispatch_mx(x, L["dst_row"], rows)
    q, s, written = O.dispatch_mxfp8(x, L["dst_row"], rows)
    assert np.array_equal(out[written], q[written])
    assert np.array_equal(sc[written], s[written])
    assert np.all(out[~written] == 0xFF) and np.all(sc[~written] == 0xFF)


def test_mxfp8_every_bf16_pattern():
    """All finite bf16 patterns, each block led by an extreme element, so
    every pattern is quantised under several shared exponents."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[np.isfinite(O.bf16_to_f32(bits))]
    rows = []
    for big in (0x43E0, 0x43FF, 0x3F80, 0x7F7F, 0x0080, 0x0001, 0x0000):
        v = np.concatenate([bits, np.zeros((-len(bits)) % 31, np.uint16)]).reshape(-1, 31)
        rows.append(np.concatenate([np.full((len(v), 1), big, np.uint16), v], axis=1).reshape(-1))
    x = np.concatenate(rows)
    x = np.concatenate([x, np.zeros((-len(x)) % 1024, np.uint16)]).reshape(-1, 1024)
    t = x.shape[0]
    out, sc = gpu_dispatch_mx(x, np.arange(t, dtype=np.int32).reshape(t, 1), t)
    q, s = O.quantize_mxfp8_blocks(x)
    assert np.array_equal(out, q) and np.array_equal(sc, s)


def test_mxfp8_layer_end_to_end():
    """DeepSeek-V3 shape with MXFP8 dispatch: route -> layout -> dispatch on
    the GPU, stand-in expert dequantises, combine against the oracle."""
    w = W.WORKLOADS["dsv3"]
    inp = W.make_inputs(w, 5)
    t = inp.x.shape[0]
    b = LayerBuffers.allocate(t, w.hidden, w.experts, w.top_k, w.ranks, 0,
                              dtype=M.MOE_DTYPE_MXFP8_E4M3)
    M.run_layer(b, dev(inp.logits), dev(inp.bias), dev(inp.x), w.score_fn, w.groups,
                w.topk_groups)
    torch.cuda.synchronize()
    idx_g, w_g = host(b.topk_idx), host(b.topk_weights)
    L = O.layout(idx_g, w.experts, w.ranks, 0)
    rows = L["num_rows"]
    q, s, written = O.dispatch_mxfp8(inp.x, L["dst_row"], rows)
    assert np.array_equal(host(b.dispatched)[:rows], q)
    assert np.array_equal(host(b.scales)[:rows], s)
    codes, sb = O.quantize_mxfp8_blocks(inp.x)
    y, _ = O.dispatch_bf16(O.expert_dequant_mx(codes, sb), L["dst_row"], rows)
    b.combine(dev(y))
    got = host(b.combined, np.uint16)[:t]
    want, _ = O.combine(y, L["dst_row"], w_g)
    assert_combine_exact(got, want, "mxfp8 layer")


# --------------------------------------------------------------- backward

BWD_CASES = [
    # T, H, k, rows, drop_frac
    (4096, 7168, 8, 32768, 0.0),
    (3000, 7040, 8, 24000, 0.1),       # dispatch backward through the held-output combine
    (1000, 520, 3, 3200, 0.1),
    (777, 4096, 6, 5000, 0.2),
    (200, 512, 11, 3000, 0.1),
    (64, 16384, 2, 300, 0.0),          # several chunk groups per wave
    (37, 8, 1, 40, 0.0),
    (0, 256, 2, 0, 0.0),
]


def _bwd_inputs(case):
    t, h, k, rows, drop = case
    g = np.random.Generator(np.random.PCG64(t + 7 * h + k))
    dst = g.permutation(max(rows, 1))[: t * k].reshape(t, k).astype(np.int32) if t else \
        np.zeros((0, k), np.int32)
    if t:
        dst[g.random((t, k)) < drop] = -1
    return g, dst


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "T%d_H%d_k%d_rows%d" % c[:4])
def test_dispatch_backward_parity(case):
    t, h, k, rows, drop = case
    say("dispatch backward case", case)
    g, dst = _bwd_inputs(case)
    grows = W.random_bf16_rows(g, rows, h)
    out_full = poison_like((max(t, 1) + GUARD, h), torch.int16)
    M.moe_dispatch_backward(t, h, k, rows, dev(grows) if rows else None,
                            dev(dst) if t else None, out_full)
    out = host(out_full, np.uint16)
    assert np.all(out[max(t, 1):] == 0xFFFF)
    want, _ = O.dispatch_backward(grows, dst)
    assert_combine_exact(out[:t], want, "dispatch backward")


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "T%d_H%d_k%d_rows%d" % c[:4])
def test_combine_backward_parity(case):
    t, h, k, rows, drop = case
    say("combine backward case", case)
    g, dst = _bwd_inputs(case)
    dout = W.random_bf16_rows(g, t, h)
    y = W.random_bf16_rows(g, rows, h)
    w = W.random_weights(g, t, k)
    dy_full = poison_like((rows + GUARD, h), torch.int16)
    dw_full = poison_like((max(t, 1), k), torch.float32)
    M.moe_combine_backward(t, h, k, rows, dev(dout) if t else None, dev(y) if rows else None,
                           dev(dst) if t else None, dev(w) if t else None, dy_full, dw_full)
    dy = host(dy_full, np.uint16)
    dw = host(dw_full)[:t]
    assert np.all(dy[rows:] == 0xFFFF), "stray write after grad_expert_out"
    want_dy, written, want_dw, dw_abs = O.combine_backward(dout, y, dst, w, rows)
    assert np.all(dy[:rows][~written] == 0xFFFF)          # rows of no pair stay untouched
    frac = assert_bf16_within_ulp(dy[:rows][written], want_dy[written], "grad_expert_out")
    live = dst >= 0
    assert np.all(dw[~live] == 0.0)
    err = np.abs(dw.astype(np.float64) - want_dw.astype(np.float64))
    assert np.all(err <= dot_tolerance(h, want_dw.astype(np.float64), dw_abs))
    say("  dy bit-exact fraction %.6f, max dw error / bound %.3g" % (
        frac, float(np.max(err / np.maximum(dot_tolerance(h, want_dw, dw_abs), 1e-30))) if t else 0))


# ------------------------------------------------------------ graph replay

def test_binding_enqueues_on_torch_current_stream():
    """Calls without a stream argument go to torch's current stream, also
    inside a `torch.cuda.stream` block."""
    assert M._stream(None) == torch.cuda.current_stream().cuda_stream
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert M._stream(None) == side.cuda_stream
        # and the work really lands there: a combine ordered after a fill
        # on the side stream sees the filled rows
        y = torch.zeros((4, 8), dtype=torch.int16, device="cuda")
        dst = torch.arange(4, dtype=torch.int32, device="cuda").view(4, 1)
        w = torch.ones((4, 1), dtype=torch.float32, device="cuda")
        out = torch.zeros((4, 8), dtype=torch.int16, device="cuda")
        y.fill_(0x3F80)                       # bf16 1.0
        M.moe_combine(4, 8, 1, 4, y, dst, w, out)
    side.synchronize()
    assert (out == 0x3F80).all()
    assert M._stream(None) == torch.cuda.current_stream().cuda_stream


def test_decode_steps_replay_in_a_graph():
    """Three decode steps (route, layout + FP8 dispatch into capacity buffers
    as one launch, combine) captured in one HIP graph; the graph is replayed three times with
    eager work and synchronisations between replays, and every replay must
    equal the eager run bit for bit."""
    w = W.WORKLOADS["decode"]
    steps = [W.make_inputs(w, w.step_seed0 + i) for i in range(3)]
    ins = [(dev(s.logits), dev(s.bias), dev(s.x)) for s in steps]
    bufs = [LayerBuffers.allocate(w.tokens, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  fp8=True) for _ in steps]
    y = dev(W.random_bf16_rows(np.random.Generator(np.random.PCG64(9)), w.num_rows, w.hidden))

    def run():
        for (lg, bi, x), b in zip(ins, bufs):
            M.run_layer(b, lg, bi, x, w.score_fn, w.groups, w.topk_groups)
            b.combine(y)

    names = ("topk_idx", "topk_weights", "dst_row", "src_pair", "expert_counts", "overflow",
             "combined")
    run()
    torch.cuda.synchronize()
    eager = [[getattr(b, n).clone() for n in names] for b in bufs]
    eager_q = [b.dispatched[b.src_pair >= 0].clone() for b in bufs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for b in bufs:                       # eager work between replays
            for n in names:
                getattr(b, n).fill_(-7 if getattr(b, n).dtype != torch.float32 else -7.0)
            b.dispatched.fill_(0x55)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for b, e, q in zip(bufs, eager, eager_q):
            for n, v in zip(names, e):
                assert torch.equal(getattr(b, n), v), (rep, n)
            assert torch.equal(b.dispatched[b.src_pair >= 0], q), rep


@pytest.mark.parametrize("shape", [
    # DeepSeek-V3-shaped layer: 32 layout tiles, packed rows, FP8 dispatch
    ("dsv3", None),
    # a smaller softmax layer with bf16 dispatch over several tiles
    ("qwen3_skew", 2048),
], ids=lambda s: s[0] if s[1] is None else "%s_T%d" % s)
def test_packed_layer_steps_replay_in_a_graph(shape):
    """Two packed multi-tile layer passes (route, count + place layout, dispatch,
    combine; each with its own inputs) captured in one HIP graph, as the
    benchmark times them. The graph is replayed three times with eager work
    and synchronisations between replays; every replay must equal the eager
    run bit for bit, and the eager layout equals the oracle's."""
    name, tokens = shape
    w = W.WORKLOADS[name]
    t = tokens or w.tokens
    say("graph replay case", name, "T=%d" % t)
    steps = [W.make_inputs(w, 11 + i, tokens=t) for i in range(2)]
    ins = [(dev(s.logits), dev(s.bias) if s.bias is not None else None, dev(s.x)) for s in steps]
    bufs = [LayerBuffers.allocate(t, w.hidden, w.experts, w.top_k, w.ranks, w.capacity,
                                  dtype=w.dispatch_dtype) for _ in steps]
    g = np.random.Generator(np.random.PCG64(21))
    y = dev(W.random_bf16_rows(g, bufs[0].num_rows, w.hidden))

    def run():
        for (lg, bi, x), b in zip(ins, bufs):
            M.run_layer(b, lg, bi, x, w.score_fn, w.groups, w.topk_groups)
            b.combine(y)

    names = ("topk_idx", "topk_weights", "dst_row", "src_pair", "expert_counts",
             "expert_offsets", "rank_counts", "rank_offsets", "rank_token_counts", "combined",
             "dispatched")
    if bufs[0].scales is not None:
        names = names + ("scales",)
    run()
    torch.cuda.synchronize()
    eager = [[getattr(b, n).clone() for n in names] for b in bufs]
    for b in bufs:
        L = O.layout(host(b.topk_idx), w.experts, w.ranks, 0)
        assert np.array_equal(host(b.dst_row), L["dst_row"])
        assert np.array_equal(host(b.expert_counts), L["expert_counts"])
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for b in bufs:                       # eager work between replays
            for n in names:
                v = getattr(b, n)
                v.fill_(-7.0 if v.dtype == torch.float32 else -7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for b, e in zip(bufs, eager):
            for n, v in zip(names, e):
                assert torch.equal(getattr(b, n), v), (rep, n)
    say("  3 replays equal the eager run")
