"""Seeded synthetic inputs for the MoE routing / dispatch / combine path.

This module only draws random numbers and shapes them. It holds none of the
method's arithmetic (no top-k, no layout, no quantisation, no reduction), so
that both the CPU oracle and the GPU path can take their inputs from here
without sharing any code with each other.

Every workload is a single MoE layer on one GPU: T tokens with hidden size H,
E experts of which each token picks k, and the E experts split into R
simulated destination ranks of E/R whole experts each (the placement rule of
the glossary page "Expert Parallelism (Parallélisme d'experts)", section
"Le principe de base": with 8 experts on 4 GPUs each GPU owns 2 of them).

Random draws use numpy's PCG64 generator, seeded per workload and step:
  * hidden states x ~ N(0, 1) drawn in fp32 and truncated to bf16 (the top 16
    bits of the fp32 pattern are kept);
  * router logits ~ N(0, 1) in fp32;
  * a per-expert bias in fp32: N(0, 0.1) for the DeepSeek-V3-shaped layers,
    a Zipf(1.2) popularity bias for the skewed Qwen3-shaped layer, none
    otherwise.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1

DTYPE_BF16 = 0
DTYPE_FP8_E4M3 = 1

# Strength of the Zipf(1.2) popularity bias of the skewed layer. It was picked
# so that, for seed 0, the busiest expert receives about ten times the mean
# load T*k/E under softmax top-8 routing; the oracle test of the workloads
# checks that property, so a change here that breaks it fails a test.
ZIPF_EXPONENT = 1.2
ZIPF_ALPHA = 0.438


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    tokens: int          # T
    hidden: int          # H
    experts: int         # E
    top_k: int           # k
    ranks: int           # R simulated destination ranks
    score_fn: int        # SCORE_SOFTMAX or SCORE_SIGMOID
    groups: int          # G expert groups (1 = plain top-k)
    topk_groups: int     # groups kept per token (1 = plain top-k)
    dispatch_dtype: int  # DTYPE_BF16 or DTYPE_FP8_E4M3
    capacity: int        # rows per expert; 0 = packed (rows = T*k)
    bias: str            # "none", "normal", "zipf"
    expert_kind: str     # stand-in expert used between dispatch and combine
    steps: int = 1       # decode: number of back-to-back steps
    step_seed0: int = 0  # decode: seed of the first step

    @property
    def experts_per_rank(self) -> int:
        return self.experts // self.ranks

    @property
    def num_rows(self) -> int:
        if self.capacity > 0:
            return self.experts * self.capacity
        return self.tokens * self.top_k


WORKLOADS = {
    "tiny": Workload("tiny", 128, 256, 8, 2, 4, SCORE_SOFTMAX, 1, 1,
                     DTYPE_BF16, 0, "none", "identity"),
    "mixtral": Workload("mixtral", 16384, 4096, 8, 2, 8, SCORE_SOFTMAX, 1, 1,
                        DTYPE_BF16, 0, "none", "scaled"),
    "dsv3": Workload("dsv3", 4096, 7168, 256, 8, 32, SCORE_SIGMOID, 8, 4,
                     DTYPE_FP8_E4M3, 0, "normal", "dequant"),
    "qwen3_skew": Workload("qwen3_skew", 8192, 4096, 128, 8, 16, SCORE_SOFTMAX,
                           1, 1, DTYPE_BF16, 0, "zipf", "identity"),
    "decode": Workload("decode", 128, 7168, 256, 8, 32, SCORE_SIGMOID, 8, 4,
                       DTYPE_FP8_E4M3, 128, "normal", "dequant",
                       steps=1000, step_seed0=1000),
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits_from_normal(gen: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) fp32 draws truncated to bf16; returned as uint16 bit patterns."""
    f = gen.standard_normal(size=shape, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def zipf_bias(gen: np.random.Generator, experts: int,
              alpha: float = ZIPF_ALPHA, s: float = ZIPF_EXPONENT) -> np.ndarray:
    """Per-expert popularity bias: a seeded permutation pi of the experts,
    popularity z_e = (pi(e)+1)^-s, bias b_e = alpha * ln(z_e / max z)."""
    perm = gen.permutation(experts)
    z = (perm.astype(np.float64) + 1.0) ** (-s)
    return (alpha * np.log(z / z.max())).astype(np.float32)


@dataclasses.dataclass
class LayerInputs:
    x: np.ndarray                 # [T, H] uint16 (bf16 bits)
    logits: np.ndarray            # [T, E] float32
    bias: Optional[np.ndarray]    # [E] float32 or None


def make_inputs(w: Workload, seed: int, tokens: Optional[int] = None) -> LayerInputs:
    """Inputs of one layer pass. `tokens` overrides T (smaller parity cases);
    the bias only depends on the seed, never on T."""
    t = w.tokens if tokens is None else tokens
    g = rng(seed)
    bias = None
    if w.bias == "normal":
        bias = (g.standard_normal(size=w.experts, dtype=np.float32)
                * np.float32(0.1)).astype(np.float32)
    elif w.bias == "zipf":
        bias = zipf_bias(g, w.experts)
    logits = g.standard_normal(size=(t, w.experts), dtype=np.float32)
    x = bf16_bits_from_normal(g, (t, w.hidden))
    return LayerInputs(x=x, logits=logits, bias=bias)


def random_topk_idx(gen: np.random.Generator, tokens: int, experts: int,
                    top_k: int, distinct: bool = True,
                    mask_frac: float = 0.0) -> np.ndarray:
    """Arbitrary routing decisions for layout tests: per token k experts,
    distinct or not, with a fraction of slots masked to -1."""
    if distinct:
        keys = gen.random((tokens, experts))
        idx = np.argsort(keys, axis=1)[:, :top_k].astype(np.int32)
    else:
        idx = gen.integers(0, experts, size=(tokens, top_k), dtype=np.int32)
    if mask_frac > 0:
        m = gen.random((tokens, top_k)) < mask_frac
        idx[m] = -1
    return idx


def random_bf16_rows(gen: np.random.Generator, rows: int, hidden: int) -> np.ndarray:
    return bf16_bits_from_normal(gen, (rows, hidden))


def random_weights(gen: np.random.Generator, tokens: int, top_k: int) -> np.ndarray:
    return gen.random((tokens, top_k), dtype=np.float32)
