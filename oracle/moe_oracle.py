"""CPU oracle of the MoE routing -> layout -> dispatch -> combine path.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import this module:
only the tests, the smoke check of the entry module and the CPU-baseline leg
of the benchmark use it. It shares no code with the HIP library and imports
nothing from it.

Every function is the plain definition of what the method computes, written
with numpy, in fp64 wherever the pages leave the floating-point precision
open. Where a floating-point value decides an integer (an expert choice, an
FP8 code) the decision is taken in fp32, the precision the GPU kernels use.

Sources (four web pages on MoE expert parallelism):
  * glossary page "Expert Parallelism (Parallélisme d'experts)" (polydesk.ai):
    section "Le principe de base" (whole experts per GPU, 8 experts on 4 GPUs
    gives 2 per GPU), section "Le pattern de communication all-to-all"
    (Phase 1 dispatch sends each token to the GPUs of its experts and each GPU
    receives the tokens of its local experts; Phase 2 combine brings results
    back and sums them weighted by the router scores), section
    "Megatron-LM (NVIDIA)" and "Défis et optimisations" (capacity factor and
    token dropping);
  * article "DeepEP de DeepSeek : la lib open source qui optimise la
    communication GPU pour les modèles MoE à l'échelle" (ai-master.dev):
    sections "Kernels low-latency dispatch et combine", "Support FP8 et
    MXFP8" (FP8 halves the bytes of BF16), "Group-limited gating algorithm"
    (each token's choice is limited to a subset of expert groups),
    "Configuration type" (dispatch/combine calls do optional FP8 quantisation);
  * the hyper.ai story on NVIDIA Hybrid-EP (single section): top-k routing,
    dispatch and combine operators, native FP8/BF16, buffers preallocated at
    a maximum size so that no size synchronisation is needed.

Readings where the pages are silent (each is also listed in the design notes):
  R1 top-k order: descending key, ties to the lower expert index.
  R2 stable slots: pairs (t, j) of one expert are placed in row-major (t, j)
     order.
  R3 group score: sum of the two largest keys of the group.
  R4 bias: enters the selection key only, never the weights.
  R5 weights: normalised over the k selected experts, no extra scale.
  R6 FP8: OCP e4m3fn, 1x128 blocks along H, scale = amax/448 in fp32, codes
     by round-to-nearest-even of x*(448/amax) with saturation to +-448.
  R7 capacity: pairs beyond `cap` in an expert's stable order are dropped.
  R14 combine arithmetic: the weighted sum is accumulated in fp32, one fused
     multiply-add per pair in slot order starting from +0, and rounded once
     to bf16 (the combine contract: fp32 accumulation in a fixed slot order);
     the same rule serves the gradient of dispatch and both levels of the
     hierarchical combine.
  R18 MXFP8: 1x32 blocks, E8M0 scale 2^(floor(log2 amax) - 8), e4m3fn codes
     of x / scale with round-to-nearest-even and saturation.
  R20 deduplicated dispatch: one row per (token, rank) with at least one
     unmasked expert there (capacity ignored), rows of a rank in token order;
     hierarchical combine: per-(token, rank) partial sums rounded to bf16,
     then a per-token sum of the partials rounded once more.
"""

from __future__ import annotations

import numpy as np

F32 = np.float32
F64 = np.float64

E4M3_MAX = 448.0


# ---------------------------------------------------------------------------
# Number formats (own codecs, defined from the bit layouts)
# ---------------------------------------------------------------------------

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (bf16 is the top half of fp32)."""
    return (bits.astype(np.uint32) << 16).view(F32)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round real values (fp32 or fp64 array) to the nearest bf16, ties to
    even, and return the bf16 bit patterns (uint16).

    bf16 keeps 8 significant bits and fp32's exponent range. The spacing of
    bf16 values around |v| is q = 2^(e-7) with 2^e <= |v| < 2^(e+1), and
    q = 2^-133 below the smallest normal 2^-126. Division and multiplication
    by q are exact in fp64, and rint() rounds half to even, so rint(v/q)*q is
    the correctly rounded bf16 value. Magnitudes that round beyond the
    largest bf16 become infinities when narrowed to fp32."""
    v = np.asarray(v, dtype=F64)
    a = np.abs(v)
    _, ex = np.frexp(a)                      # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -126)             # floor(log2 a), clamped to subnormals
    q = np.ldexp(np.ones_like(a), e - 7)
    r = np.rint(a / q) * q
    r = np.where(a == 0, 0.0, r)
    with np.errstate(over="ignore"):
        r32 = np.copysign(r, v).astype(F32)
    r32 = np.where(np.isnan(v), np.float32(np.nan), r32)
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def e4m3_decode_table() -> np.ndarray:
    """Value of each of the 256 OCP e4m3fn codes: 1 sign bit, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent field 0 encodes subnormals m*2^-9;
    0x7F and 0xFF are NaN; there are no infinities."""
    vals = np.empty(256, dtype=F64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        m = code & 0x7
        if ef == 0xF and m == 0x7:
            vals[code] = np.nan
        elif ef == 0:
            vals[code] = s * m * 2.0 ** -9
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return vals


_E4M3_TABLE = e4m3_decode_table()
_E4M3_POS = _E4M3_TABLE[:0x7F]               # codes 0x00..0x7E, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3_TABLE[codes.astype(np.intp)]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3fn codes (uint8), round to nearest, ties to even,
    magnitudes above 448 saturate to 448, the sign is kept (also of zero).

    e4m3 spacing around |v| is q = 2^(e-3) for 2^e <= |v| < 2^(e+1) with
    e >= -6, and 2^-9 below 2^-6. rint(|v|/q)*q is the nearest e4m3 value
    with ties to even, because the code's last bit is the mantissa's last
    bit. The result is looked up in the table of positive codes."""
    v = np.asarray(v, dtype=F32).astype(F64)
    a = np.abs(v)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    q = np.ldexp(np.ones_like(a), e - 3)
    r = np.minimum(np.rint(a / q) * q, E4M3_MAX)
    r = np.where(a == 0, 0.0, r)
    mag = np.searchsorted(_E4M3_POS, r).astype(np.uint8)
    sign = np.where(np.signbit(v), 0x80, 0x00).astype(np.uint8)
    return mag | sign


# ---------------------------------------------------------------------------
# Routing (top-k and group-limited top-k)
# ---------------------------------------------------------------------------

def _sigmoid_f32(logits: np.ndarray) -> np.ndarray:
    """Router score 1/(1+exp(-l)) evaluated in fp64 and rounded once to fp32."""
    l64 = logits.astype(F64)
    return (1.0 / (1.0 + np.exp(-l64))).astype(F32)


def _selection_key(score: np.ndarray, bias) -> np.ndarray:
    """Selection key = score + bias (fp32 add); the bias only moves the
    choice, never the weights (reading R4)."""
    if bias is None:
        return score.astype(F32)
    return (score.astype(F32) + np.asarray(bias, dtype=F32)[None, :]).astype(F32)


def _top_k_order(key: np.ndarray, allowed=None) -> np.ndarray:
    """Expert indices of each row sorted by (allowed first, key descending,
    index ascending) (reading R1)."""
    t, e = key.shape
    idx = np.broadcast_to(np.arange(e), (t, e))
    keys = [idx, -key.astype(F64)]
    if allowed is not None:
        keys.append(~allowed)
    return np.lexsort(keys, axis=-1)


def route_softmax_topk(logits: np.ndarray, top_k: int, bias=None):
    """Softmax top-k routing (hyper.ai story on Hybrid-EP: each token activates
    only k experts; glossary "Expert Parallelism", Phase 2: outputs are
    weighted by the router scores).

    Selection: the k largest keys l_e + b_e. Weights: softmax of the raw
    logits restricted to the selected experts, w_j = exp(l_j)/sum_i exp(l_i),
    in fp64 and rounded once to fp32 (reading R5)."""
    logits = np.asarray(logits, dtype=F32)
    key = _selection_key(logits, bias)
    sel = _top_k_order(key)[:, :top_k].astype(np.int32)
    l_sel = np.take_along_axis(logits, sel, axis=1).astype(F64)
    m = l_sel.max(axis=1, keepdims=True)
    u = np.exp(l_sel - m)
    w = (u / u.sum(axis=1, keepdims=True)).astype(F32)
    return sel, w


def group_scores(key: np.ndarray, num_groups: int) -> np.ndarray:
    """Score of each contiguous expert group: the sum, in fp32, of the two
    largest selection keys in the group, largest first (reading R3). A group
    of one expert scores that expert's key."""
    t, e = key.shape
    g = key.reshape(t, num_groups, e // num_groups)
    srt = np.sort(g, axis=2)
    if srt.shape[2] == 1:
        return srt[:, :, 0].astype(F32)
    return (srt[:, :, -1] + srt[:, :, -2]).astype(F32)


def kept_groups(gscore: np.ndarray, topk_groups: int) -> np.ndarray:
    """Boolean [T, G]: the topk_groups best groups, ties to the lower group."""
    order = _top_k_order(gscore)[:, :topk_groups]
    keep = np.zeros(gscore.shape, dtype=bool)
    np.put_along_axis(keep, order, True, axis=1)
    return keep


def route_group_limited(logits: np.ndarray, top_k: int, num_groups: int,
                        topk_groups: int, bias=None):
    """Group-limited sigmoid top-k (DeepEP article, section "Group-limited
    gating algorithm": a token chooses among the experts of a few groups
    only, which bounds its set of destinations).

    1. s_e = sigmoid(l_e) in fp64, rounded to fp32; key_e = s_e + b_e (fp32).
    2. Group score = sum of the group's two largest keys.
    3. Keep the `topk_groups` best groups.
    4. Select the k largest keys among experts of kept groups.
    5. w_j = s_j / sum_i s_i over the selected experts (fp64, rounded once)."""
    logits = np.asarray(logits, dtype=F32)
    t, e = logits.shape
    s = _sigmoid_f32(logits)
    key = _selection_key(s, bias)
    keep_g = kept_groups(group_scores(key, num_groups), topk_groups)
    allowed = np.repeat(keep_g, e // num_groups, axis=1)
    sel = _top_k_order(key, allowed)[:, :top_k].astype(np.int32)
    s_sel = np.take_along_axis(s, sel, axis=1).astype(F64)
    w = (s_sel / s_sel.sum(axis=1, keepdims=True)).astype(F32)
    return sel, w


def route(logits, top_k, score_fn, num_groups=1, topk_groups=1, bias=None):
    """score_fn 0 = softmax top-k, 1 = sigmoid (group-limited when G > 1)."""
    if score_fn == 0:
        if num_groups != 1:
            raise ValueError("softmax routing takes no groups")
        return route_softmax_topk(logits, top_k, bias)
    return route_group_limited(logits, top_k, num_groups, topk_groups, bias)


# ---------------------------------------------------------------------------
# Layout: counts, offsets and the stable slot of every (token, slot) pair
# ---------------------------------------------------------------------------

def layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int,
           capacity: int = 0) -> dict:
    """Counts, prefix-sum offsets and stable destination rows.

    Placement (glossary "Expert Parallelism", "Le principe de base"): rank r
    owns the whole experts [r*E/R, (r+1)*E/R). Dispatch (same page, Phase 1)
    sends each pair to the region of its expert's rank; here the ranks are
    consecutive regions of one buffer, ordered by expert.

    Packed mode (capacity 0), buffers of T*k rows sized in advance so that no
    count has to be read back first (hyper.ai story on Hybrid-EP):
      count_e  = number of pairs (t, j) with idx[t, j] = e (masked -1 skipped)
      offset_e = sum of count_e' for e' < e
      dst_row[t, j] = offset_e + number of earlier pairs of expert e in
                      row-major (t, j) order (reading R2)
    Capacity mode (cap > 0; glossary sections "Megatron-LM (NVIDIA)" and
    "Défis et optimisations", capacity factor and token dropping): the pair
    with stable position p in expert e goes to row e*cap + p if p < cap and
    is dropped (-1) otherwise (reading R7).

    rank_counts[r] counts the rows written into rank r's region;
    rank_token_counts[r] counts the distinct tokens with at least one
    selected (unmasked) expert on rank r; src_pair is the inverse map
    row -> t*k + j, -1 on rows that receive nothing."""
    idx = np.asarray(topk_idx, dtype=np.int64)
    t, k = idx.shape
    e_cnt, r_cnt = num_experts, num_ranks
    epr = e_cnt // r_cnt
    flat = idx.reshape(-1)
    pairs = np.nonzero(flat >= 0)[0]            # row-major order of live pairs
    experts = flat[pairs]

    counts = np.bincount(experts, minlength=e_cnt).astype(np.int64)
    starts = np.concatenate([[0], np.cumsum(counts)])

    # stable position of each live pair inside its expert: stable sort by
    # expert keeps the row-major order among pairs of the same expert
    order = np.argsort(experts, kind="stable")
    pos = np.empty(len(pairs), dtype=np.int64)
    pos[order] = np.arange(len(pairs)) - starts[experts[order]]

    dst = np.full(t * k, -1, dtype=np.int64)
    if capacity == 0:
        rows = t * k
        dst[pairs] = starts[experts] + pos
        offsets = starts
        kept = counts
        overflow = 0
    else:
        rows = e_cnt * capacity
        keep = pos < capacity
        dst[pairs[keep]] = experts[keep] * capacity + pos[keep]
        offsets = np.arange(e_cnt + 1, dtype=np.int64) * capacity
        kept = np.minimum(counts, capacity)
        overflow = int(np.maximum(counts - capacity, 0).sum())

    src = np.full(rows, -1, dtype=np.int64)
    live = dst >= 0
    src[dst[live]] = np.nonzero(live)[0]

    rank_counts = kept.reshape(r_cnt, epr).sum(axis=1)
    rank_offsets = offsets[::epr]

    tok = pairs // k
    tr = np.unique(tok * r_cnt + experts // epr)
    rank_token_counts = np.bincount(tr % r_cnt, minlength=r_cnt)

    i32 = np.int32
    return dict(
        expert_counts=counts.astype(i32),
        expert_offsets=offsets.astype(i32),
        rank_counts=rank_counts.astype(i32),
        rank_offsets=rank_offsets.astype(i32),
        rank_token_counts=rank_token_counts.astype(i32),
        dst_row=dst.reshape(t, k).astype(i32),
        src_pair=src.astype(i32),
        overflow=np.array([overflow], dtype=i32),
        num_rows=rows,
    )


# ---------------------------------------------------------------------------
# Dispatch: permute bf16 rows into the expert-ordered buffer (optionally FP8)
# ---------------------------------------------------------------------------

def dispatch_bf16(x_bits: np.ndarray, dst_row: np.ndarray, num_rows: int):
    """out[dst_row[t, j]] = x[t] for every pair that has a row (glossary
    "Expert Parallelism", Phase 1). Returns (out, written) where `written`
    marks the rows that received a token; other rows are left undefined."""
    t, h = x_bits.shape
    out = np.zeros((num_rows, h), dtype=np.uint16)
    written = np.zeros(num_rows, dtype=bool)
    d = dst_row.reshape(-1)
    tok = np.repeat(np.arange(t), dst_row.shape[1])
    live = d >= 0
    out[d[live]] = x_bits[tok[live]]
    written[d[live]] = True
    return out, written


FP8_BLOCK = 128


def fp8_block_scale_inv(x_bits: np.ndarray):
    """Per token and 128-column block: a = max |x| (exact in fp32), the stored
    scale fp32(a / 448) and the multiplier fp32(448 / a) (+inf when a = 0 or
    when the quotient overflows fp32)."""
    t, h = x_bits.shape
    xf = bf16_to_f32(x_bits).reshape(t, h // FP8_BLOCK, FP8_BLOCK)
    a = np.abs(xf).max(axis=2)
    with np.errstate(divide="ignore", over="ignore"):
        scale = (a / F32(E4M3_MAX)).astype(F32)
        inv = (F32(E4M3_MAX) / a).astype(F32)
    return scale, inv


def quantize_fp8_blocks(x_bits: np.ndarray):
    """Per-token, per-128-column FP8 quantisation of bf16 rows (DeepEP article,
    "Support FP8 et MXFP8": FP8 payloads halve the BF16 bytes; hyper.ai story
    on Hybrid-EP: native FP8 in dispatch; reading R6). For each block:
        a     = max |x|                     (exact)
        scale = fp32(a / 448)
        inv   = fp32(448 / a)
        q     = e4m3(fp32(x * inv)),  q = signed zero where x = +-0
    Returns codes [T, H] uint8 and scales [T, H/128] fp32."""
    t, h = x_bits.shape
    nb = h // FP8_BLOCK
    xf = bf16_to_f32(x_bits).reshape(t, nb, FP8_BLOCK)
    scale, inv = fp8_block_scale_inv(x_bits)
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (xf * inv[:, :, None]).astype(F32)
    prod = np.where(xf == 0, xf, prod)       # zeros keep their sign, no NaN
    codes = e4m3_encode(prod).reshape(t, h)
    return codes, scale


def dispatch_fp8(x_bits: np.ndarray, dst_row: np.ndarray, num_rows: int):
    """FP8 dispatch: quantise each token once, copy codes and scales to every
    row of the token. Returns (codes [rows, H], scales [rows, H/128], written)."""
    t, h = x_bits.shape
    codes, scale = quantize_fp8_blocks(x_bits)
    out = np.zeros((num_rows, h), dtype=np.uint8)
    out_s = np.zeros((num_rows, h // FP8_BLOCK), dtype=F32)
    written = np.zeros(num_rows, dtype=bool)
    d = dst_row.reshape(-1)
    tok = np.repeat(np.arange(t), dst_row.shape[1])
    live = d >= 0
    out[d[live]] = codes[tok[live]]
    out_s[d[live]] = scale[tok[live]]
    written[d[live]] = True
    return out, out_s, written


# ---------------------------------------------------------------------------
# MXFP8 dispatch: 1x32 blocks with power-of-two (E8M0) scales
# ---------------------------------------------------------------------------

MX_BLOCK = 32
E8M0_BIAS = 127
E4M3_EMAX = 8          # exponent of e4m3fn's largest binade (448 = 1.75 * 2^8)


def mxfp8_block_exponents(x_bits: np.ndarray) -> np.ndarray:
    """Shared exponent of each 32-column block (DeepEP article, "Support FP8
    et MXFP8", names MXFP8; its block and scale layout is read from the OCP
    microscaling format, reading R18): e = floor(log2(max |x|)) - 8, clamped
    to the E8M0 range [-127, 127]; an all-zero block takes -127."""
    t, h = x_bits.shape
    xf = bf16_to_f32(x_bits).reshape(t, h // MX_BLOCK, MX_BLOCK).astype(F64)
    a = np.abs(xf).max(axis=2)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    e = (ex - 1) - E4M3_EMAX
    e = np.where(a == 0, -E8M0_BIAS, e)
    return np.clip(e, -E8M0_BIAS, E8M0_BIAS).astype(np.int64)


def quantize_mxfp8_blocks(x_bits: np.ndarray):
    """MXFP8 quantisation of bf16 rows: per 32-column block a power-of-two
    scale 2^e (stored as the E8M0 byte e + 127) and e4m3fn codes of x / 2^e,
    rounded to nearest even and saturated at +-448 (the division by a power
    of two is exact). Returns codes [T, H] uint8, scale bytes [T, H/32]."""
    t, h = x_bits.shape
    e = mxfp8_block_exponents(x_bits)
    xf = bf16_to_f32(x_bits).reshape(t, h // MX_BLOCK, MX_BLOCK).astype(F64)
    scaled = np.ldexp(xf, -e[:, :, None])
    codes = e4m3_encode(scaled.astype(F32)).reshape(t, h)
    return codes, (e + E8M0_BIAS).astype(np.uint8)


def dispatch_mxfp8(x_bits: np.ndarray, dst_row: np.ndarray, num_rows: int):
    """MXFP8 dispatch: quantise each token once, copy codes and scale bytes
    to every row of the token. Returns (codes, scale bytes, written)."""
    t, h = x_bits.shape
    codes, sbytes = quantize_mxfp8_blocks(x_bits)
    out = np.zeros((num_rows, h), dtype=np.uint8)
    out_s = np.zeros((num_rows, h // MX_BLOCK), dtype=np.uint8)
    written = np.zeros(num_rows, dtype=bool)
    d = dst_row.reshape(-1)
    tok = np.repeat(np.arange(t), dst_row.shape[1])
    live = d >= 0
    out[d[live]] = codes[tok[live]]
    out_s[d[live]] = sbytes[tok[live]]
    written[d[live]] = True
    return out, out_s, written


def expert_dequant_mx(codes: np.ndarray, sbytes: np.ndarray) -> np.ndarray:
    """y = bf16(decode(q) * 2^(s - 127)) for MXFP8 rows (exact product)."""
    r, h = codes.shape
    v = e4m3_decode(codes).reshape(r, h // MX_BLOCK, MX_BLOCK)
    p = np.ldexp(v, sbytes.astype(np.int64)[:, :, None] - E8M0_BIAS)
    return round_to_bf16(p.reshape(r, h))


# ---------------------------------------------------------------------------
# Combine: weighted sum of each token's expert outputs
# ---------------------------------------------------------------------------

def fma_f32(a, b, c) -> np.ndarray:
    """fp32 fused multiply-add, elementwise: a*b + c computed exactly and
    rounded once to fp32 (nearest, ties to even), for fp32 inputs.

    The product of two fp32 values has at most 48 significant bits, so it is
    exact in fp64. The sum p + c is formed in fp64 together with its exact
    rounding error (Knuth's two-sum), so that p + c = s + e exactly. Rounding
    s to fp32 is then the correct rounding of p + c, except in one case: s
    lies exactly halfway between two fp32 values while e is not zero. The
    exact sum is then off the midpoint on the side of e, and the result is
    the fp32 neighbour on that side (fp32 midpoints are fp64 numbers, so the
    fp64 rounding of p + c can land on one but never step over one)."""
    a64 = np.asarray(a, dtype=F32).astype(F64)
    b64 = np.asarray(b, dtype=F32).astype(F64)
    c64 = np.asarray(c, dtype=F32).astype(F64)
    with np.errstate(over="ignore", invalid="ignore"):   # inf and nan inputs propagate
        p = a64 * b64
        s = p + c64
        bv = s - p
        e = (p - (s - bv)) + (c64 - bv)
        r = s.astype(F32)
        r64 = r.astype(F64)
        side = np.where(s > r64, np.float32(np.inf), np.float32(-np.inf))
        n = np.nextafter(r, side)
        tie = (s != r64) & np.isfinite(r64) & (s - r64 == n.astype(F64) - s)
        fix = tie & (e != 0) & ((e > 0) == (s > r64))
    return np.where(fix, n, r).astype(F32)


def combine(y_bits: np.ndarray, dst_row: np.ndarray, topk_w: np.ndarray):
    """out[t] = bf16( sum_j w[t, j] * y[dst_row[t, j]] ) over the pairs that
    have a row (glossary "Expert Parallelism", Phase 2: results return to the
    token's origin and are summed weighted by the router scores).

    The sum is accumulated in fp32 in slot order, one fused multiply-add per
    pair: acc = +0; for j = 0..k-1 with a row, acc = fma_f32(w[t, j],
    y[dst_row[t, j]], acc); then acc is rounded to bf16 (nearest even).
    Dropped pairs add nothing and the weights are not renormalised.
    Returns (out bits [T, H] uint16, abs_sum [T, H] fp64 = sum_j |w y|)."""
    t, k = dst_row.shape
    h = y_bits.shape[1]
    acc = np.zeros((t, h), dtype=F32)
    mag = np.zeros((t, h), dtype=F64)
    for j in range(k):
        d = dst_row[:, j]
        live = d >= 0
        if not live.any():
            continue
        yj = bf16_to_f32(y_bits[d[live]])
        wj = topk_w[live, j].astype(F32)[:, None]
        acc[live] = fma_f32(wj, yj, acc[live])
        mag[live] += np.abs(wj.astype(F64) * yj.astype(F64))
    return round_to_bf16(acc), mag


# ---------------------------------------------------------------------------
# Backward of dispatch and combine (the pages note that the exchanges run in
# both the forward and the backward pass: DeepEP article, "Qu'est-ce que
# l'Expert Parallelism", and its fine-tuning use case)
# ---------------------------------------------------------------------------

def dispatch_backward(grad_rows_bits: np.ndarray, dst_row: np.ndarray):
    """Gradient of dispatch with respect to x: each token collects the
    gradients of its rows, dx[t] = bf16( sum_j g[dst_row[t, j]] ) (the
    adjoint of copying x[t] to k rows). It is combine with unit weights: an
    fp32 sum in slot order (fma with weight 1), rounded once to bf16.
    Returns (dx bits [T, H], abs_sum [T, H])."""
    t, k = dst_row.shape
    return combine(grad_rows_bits, dst_row, np.ones((t, k), dtype=F32))


def combine_backward(grad_out_bits: np.ndarray, y_bits: np.ndarray,
                     dst_row: np.ndarray, topk_w: np.ndarray, num_rows: int):
    """Gradients of out[t] = sum_j w[t, j] * y[dst_row[t, j]]:
        dy[dst_row[t, j]] = bf16( w[t, j] * dout[t] )
        dw[t, j]          = fp32( sum_h dout[t, h] * y[dst_row[t, j], h] )
    both exact in fp64 before the final rounding. Dropped pairs (row -1)
    give dw = 0 and write no row.
    Returns (dy bits [rows, H], written, dw [T, k] fp32, dw_abs [T, k] fp64 =
    sum_h |dout * y|)."""
    t, k = dst_row.shape
    h = grad_out_bits.shape[1]
    g = bf16_to_f32(grad_out_bits).astype(F64)
    dy = np.zeros((num_rows, h), dtype=np.uint16)
    written = np.zeros(num_rows, dtype=bool)
    dw = np.zeros((t, k), dtype=F64)
    dw_abs = np.zeros((t, k), dtype=F64)
    for j in range(k):
        d = dst_row[:, j]
        live = d >= 0
        rows = d[live]
        yj = bf16_to_f32(y_bits[rows]).astype(F64)
        prod = g[live] * yj
        dw[live, j] = prod.sum(axis=1)
        dw_abs[live, j] = np.abs(prod).sum(axis=1)
        dy[rows] = round_to_bf16(topk_w[live, j].astype(F64)[:, None] * g[live])
        written[rows] = True
    return dy, written, dw.astype(F32), dw_abs


# ---------------------------------------------------------------------------
# Deduplicated dispatch and hierarchical combine (hyper.ai story on Hybrid-EP:
# the combine reduces hierarchically, first the results inside one
# destination, then across destinations). One row per (token, destination
# rank) crosses to a rank however many of its experts the token chose there;
# the rank fans the row out to its local experts, reduces their weighted
# outputs into one partial row per (token, rank), and only the partials
# travel back, where each token sums its partials (reading R20).
# ---------------------------------------------------------------------------

def rank_layout(topk_idx: np.ndarray, num_experts: int, num_ranks: int) -> dict:
    """Rows of the (token, rank) buffer.

    A token t has a row on rank r when at least one of its unmasked experts
    lives on r (rank r owns experts [r*E/R, (r+1)*E/R); glossary "Expert
    Parallelism", "Le principe de base"). Capacity plays no part: the row
    exists by demand. Rank r's rows form the region
    [rank_token_offsets[r], rank_token_offsets[r+1]) and are ordered by token
    (reading R2 applied to (token, rank) pairs). The buffer is sized for
    T * min(k, R) rows, its largest possible size, so that nothing is read
    back first (hyper.ai story on Hybrid-EP, preallocated buffers).

    Returns
      rank_token_counts [R], rank_token_offsets [R+1]
      rank_row [T, k]: the (t, rank of expert j) row of every unmasked slot,
                       -1 for masked slots
      send_row [T, k]: that row at the first slot (in slot order) of each
                       rank, -1 at the token's later slots on the same rank
                       and at masked slots; dispatching x with send_row as
                       the destination map sends one copy per (token, rank)
      row_token [T * min(k, R)]: token of each row, -1 past the last row
      num_rank_rows: T * min(k, R)"""
    idx = np.asarray(topk_idx, dtype=np.int64)
    t, k = idx.shape
    epr = num_experts // num_ranks
    live = (idx >= 0) & (idx < num_experts)
    rank = np.where(live, idx // epr, -1)

    # first slot of each (token, rank)
    first = live.copy()
    for j in range(k):
        for o in range(j):
            first[:, j] &= rank[:, o] != rank[:, j]

    hit = np.zeros((t, num_ranks), dtype=bool)
    tt, jj = np.nonzero(live)
    hit[tt, rank[tt, jj]] = True
    counts = hit.sum(axis=0).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    # position of token t among the tokens of rank r, in token order
    pos = np.cumsum(hit, axis=0) - 1
    row_of = offsets[:-1][None, :] + pos

    rank_row = np.full((t, k), -1, dtype=np.int64)
    rank_row[tt, jj] = row_of[tt, rank[tt, jj]]
    send_row = np.where(first, rank_row, -1)

    num_rank_rows = t * min(k, num_ranks)
    row_token = np.full(num_rank_rows, -1, dtype=np.int64)
    ht, hr = np.nonzero(hit)
    row_token[row_of[ht, hr]] = ht

    i32 = np.int32
    return dict(rank_token_counts=counts.astype(i32), rank_token_offsets=offsets.astype(i32),
                rank_row=rank_row.astype(i32), send_row=send_row.astype(i32),
                row_token=row_token.astype(i32), num_rank_rows=num_rank_rows)


def expand_rows(rank_rows: np.ndarray, rank_row: np.ndarray, src_pair: np.ndarray):
    """On the receiving rank, each expert row takes the (token, rank) row of
    its pair: out[q] = rank_rows[rank_row.flat[src_pair[q]]] for every row q
    that holds a pair. `rank_rows` may be bf16 bits, FP8 codes or a scale
    array: any array whose first axis is the row. Returns (out, written);
    rows without a pair are left undefined (zero here)."""
    n = src_pair.shape[0]
    out = np.zeros((n,) + rank_rows.shape[1:], dtype=rank_rows.dtype)
    written = src_pair >= 0
    flat = rank_row.reshape(-1)
    out[written] = rank_rows[flat[src_pair[written]]]
    return out, written


def combine_local(y_bits: np.ndarray, dst_row: np.ndarray, rank_row: np.ndarray,
                  topk_w: np.ndarray, num_rank_rows: int):
    """First level of the hierarchical combine: each rank reduces, for every
    token it holds a row of, the weighted outputs of that token's experts on
    the rank:
        partial[rank_row[t, j]] = bf16( sum over slots j' of t with
            rank_row[t, j'] = rank_row[t, j] and a kept expert row of
            w[t, j'] * y[dst_row[t, j']] )
    accumulated as combine() does: in fp32, one fused multiply-add per pair,
    in slot order, starting from +0, then rounded to bf16 (the partial
    travels as a bf16 row, reading R20). A (token, rank) row whose pairs
    were all dropped by capacity is still written, as +0.
    Returns (partial bits [num_rank_rows, H], written, abs_sum [num_rank_rows,
    H] = sum of |w y| of the row's terms)."""
    t, k = dst_row.shape
    h = y_bits.shape[1]
    acc = np.zeros((num_rank_rows, h), dtype=F32)
    mag = np.zeros((num_rank_rows, h), dtype=F64)
    written = np.zeros(num_rank_rows, dtype=bool)
    for j in range(k):
        s = rank_row[:, j]
        has = s >= 0
        written[s[has]] = True
        keep = has & (dst_row[:, j] >= 0)
        if not keep.any():
            continue
        wj = topk_w[keep, j].astype(F32)[:, None]
        yj = bf16_to_f32(y_bits[dst_row[keep, j]])
        # a (token, rank) row appears at most once in one slot column (the
        # rows of different tokens differ), so each row takes one step here
        # and its steps run in slot order
        rows = s[keep]
        acc[rows] = fma_f32(wj, yj, acc[rows])
        mag[rows] += np.abs(wj.astype(F64) * yj.astype(F64))
    return round_to_bf16(acc), written, mag


def combine_partials(partial_bits: np.ndarray, send_row: np.ndarray):
    """Second level: out[t] = bf16( sum over t's (token, rank) rows of the
    partial rows ), accumulated in fp32 in slot order as combine() does with
    unit weights. Each row is named once, at the rank's first slot
    (send_row). Returns (out bits [T, H], abs_sum)."""
    t, k = send_row.shape
    return combine(partial_bits, send_row, np.ones((t, k), dtype=F32))


def combine_hierarchical(y_bits: np.ndarray, dst_row: np.ndarray, topk_w: np.ndarray,
                         rank_lay: dict):
    """Both levels: the per-rank partials, then their sum per token.
    Returns (out bits [T, H], partial bits, partial abs_sum)."""
    partial, _, pmag = combine_local(y_bits, dst_row, rank_lay["rank_row"], topk_w,
                                     rank_lay["num_rank_rows"])
    out, _ = combine_partials(partial, rank_lay["send_row"])
    return out, partial, pmag


# ---------------------------------------------------------------------------
# Stand-in experts used between dispatch and combine (harness, not the method)
# ---------------------------------------------------------------------------

def expert_of_rows(expert_offsets: np.ndarray, num_rows: int) -> np.ndarray:
    """Expert that owns each row of the dispatched buffer."""
    rows = np.arange(num_rows)
    return np.searchsorted(expert_offsets[1:], rows, side="right")


def expert_scaled(out_bits: np.ndarray, expert_offsets: np.ndarray,
                  num_experts: int) -> np.ndarray:
    """y = bf16(x * (e+1)/E) for rows of expert e (exact product, one RNE)."""
    e = expert_of_rows(expert_offsets, out_bits.shape[0])
    c = (e + 1).astype(F64) / num_experts
    return round_to_bf16(bf16_to_f32(out_bits).astype(F64) * c[:, None])


def expert_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """y = bf16(fp32(decode(q) * scale)) for FP8 rows."""
    r, h = codes.shape
    v = e4m3_decode(codes).astype(F32).reshape(r, h // FP8_BLOCK, FP8_BLOCK)
    p = (v * scales[:, :, None].astype(F32)).astype(F32)
    return round_to_bf16(p.reshape(r, h))
